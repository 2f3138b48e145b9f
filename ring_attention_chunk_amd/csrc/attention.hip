// attention.hip -- chunk-statistics and ring-attention kernels for gfx950 (CDNA4).
//
// What is computed (exercise page "systems-distributed-ring-attention-online-
// softmax", problem statement and hints; "Ring Attention: Distributed Reads with
// Online Softmax", sections "A simple forward schedule" and "Causal masks depend
// on global positions"): for every query row, a running online-softmax state
// (row max m, denominator l, un-normalised numerator u) is carried across the
// keys of all chunks in list order; each new block of keys is merged by
// rescaling both sides to the shared new max; the output u / l is formed once.
//
// Mapping onto the chip
// ---------------------
//  * One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows. The workgroup walks key tiles of 64 keys in the order of the
//    concatenated chunk list, so tile boundaries never depend on how the
//    sequence was split into chunks: the result is bit-identical for any split.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l then holds one query (l % 32) and 16 of
//    the 32 keys of a block, so the row max and row sum are in-lane reductions
//    plus one exchange with lane l ^ 32. The probabilities stay in registers
//    and feed O^T = V^T P^T directly as the B operand.
//  * bf16 (attention_bf16_kernel): each wave software-pipelines its own work,
//    issuing the MFMAs of the next tile's scores between the vector
//    instructions of the current tile's softmax, and the current tile's P V
//    between the next tile's row maxima. K and V tiles are copied from HBM
//    straight into swizzled LDS rings several tiles ahead; V is read transposed
//    by the LDS itself.
//  * fp32, and bf16 inputs the pipelined path cannot copy whole 16-byte pieces
//    of (attention_kernel): one tile per iteration, the next tile fetched from
//    HBM into registers while the current one is computed, then stored to
//    double-buffered LDS (V transposed).
//  * With a causal mask, tiles and whole chunks whose keys lie after every
//    query of the workgroup are skipped; tiles with a mix of visible and hidden
//    keys are masked per element (positions, never local indices).
//  * When (batch x heads x query tiles) is too small to fill the chip, the key
//    tiles are cut into equal ranges handled by separate workgroups; their
//    partial (u, l, m) are merged in range order by a second kernel. The cut
//    depends only on the number of keys, never on the chunk list.
//  * The merge of two statistics is a separate bandwidth-bound kernel.

#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ring_attention_chunk.h"
#include "host_common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
// Keys per tile: 128 halves the per-tile costs (barrier, copy issue, tile
// walk) relative to the matrix work; 64 at head_dim 128 for registers.
constexpr int pipe_tile(int dp) { return dp == 128 ? 64 : 128; }
constexpr int BN = 64;           // keys per tile
constexpr int kPosNone = 0x7fffffff;      // position of a missing key: after everything
constexpr int kPosAll = 0x7ffffffe;       // query position that allows every real key
constexpr int kPosMin = -0x7fffffff - 1;  // query position of a missing row
constexpr float kLog2e = 1.4426950408889634f;

enum Mode { kStats = 0, kRingFull = 1, kRingCausal = 2 };

// Pipelined bf16 kernel: waves per workgroup, by mode; always two waves per
// SIMD. The ring calls use eight-wave workgroups (256 query rows): one K/V
// ring per CU instead of two halves the copies into LDS, and the L2 traffic,
// per flop. The chunk-statistics call keeps four-wave workgroups: it has no
// key-range split, and 256-row workgroups would leave half the CUs idle on
// short query shares.
constexpr int pipe_waves(int mode) { return mode == kStats ? 4 : 8; }
constexpr int pipe_bm(int mode) { return 32 * pipe_waves(mode); }
constexpr int pipe_resident(int mode) { return 8 / pipe_waves(mode); }

// Chunk descriptor as the kernels read it (64 bytes).
struct ChunkDev {
  const void* k;
  const void* v;
  int64_t start;  // index of the chunk's first key in the concatenated list
  int64_t len;
  int64_t sb, sh, ss;
  int32_t pos0;  // global position of the first key
  int32_t ps;    // position step between consecutive keys (1: contiguous; P: striped over P devices)
};

struct QSegDev {
  int64_t row0;
  int64_t len;
  int64_t pos0;
  int64_t ps;  // position step between consecutive rows
};
static_assert(sizeof(ChunkDev) % 4 == 0 && sizeof(QSegDev) % 4 == 0, "tables are uploaded in 4-byte words");

struct Params {
  const void* q;
  float* o;    // out (ring) or u (stats)
  float* l;    // lse (ring, may be null) or l (stats)
  float* m;    // m (stats)
  float* part; // split partials: u [nsplit][rows][d], then l and m [nsplit][rows]
  const ChunkDev* chunks;
  const QSegDev* qsegs;
  ChunkDev one;  // the single chunk of the stats call
  int64_t Lq, Lk;
  int n_chunks, n_qseg;
  int B, Hq, Hkv, d;
  int n_qt;
  int nsplit;   // key-tile ranges per (batch, head, query tile)
  int vec;      // 16-byte loads allowed for q, k and v
  int kps;      // position step shared by every chunk (pipelined causal path only)
  double kinv;  // 1 / kps
  float scale;  // softmax scale
  float c2;     // scale * log2(e)
  // block-sparse calls: per query tile, the ascending list of key tiles that hold
  // a visible pair (sp_count entries of the row of sp_cap), and the block mask
  // packed 32 key blocks per word, sp_rw words per query block
  const int* sp_list;
  const int* sp_count;
  const uint32_t* sp_bits;
  int sp_cap, sp_rw;
  int sp_lgq, sp_lgk;  // log2 of the query and key block sizes (positions)
};

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 with no operand
// canonicalisation, unlike fmaxf.
__device__ __forceinline__ float fmax_raw(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum of x over lanes l and l ^ 32, on every lane, via v_permlane32_swap.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lazy rescaling: the running numerator and denominator stay relative to a
// reference maximum until a score exceeds it by more than 2^kLazy (in exp2
// units), so most tiles need no rescale of u. u/l and ref + log(l) do not
// depend on the reference; the chunk-stats call converts to the true maximum
// at the end.
constexpr float kLazy = 8.0f;

// Loads through global-address-space pointers. Pointers read from the chunk
// table carry no address space; generic (flat) loads would also count against
// the LDS wait counter and make every LDS wait drain the HBM prefetch.
typedef const u32x4 __attribute__((address_space(1)))* gptr_u32x4;
typedef const uint16_t __attribute__((address_space(1)))* gptr_u16;
typedef const float __attribute__((address_space(1)))* gptr_f32;
__device__ __forceinline__ u32x4 gload16(const void* ptr) { return *(gptr_u32x4)ptr; }
__device__ __forceinline__ uint32_t gload_u16(const void* ptr) { return *(gptr_u16)ptr; }
__device__ __forceinline__ float gload_f32(const void* ptr) { return *(gptr_f32)ptr; }

// Chunk descriptors are read through the constant address space: with the
// walk's uniform cursor these are scalar loads, which leave the vector memory
// counter (that the LDS copy pipeline waits on) alone.
typedef const __attribute__((address_space(4))) ChunkDev* cchunk_ptr;
template <int MODE>
__device__ __forceinline__ ChunkDev chunk_at(const Params& p, int c) {
  if constexpr (MODE == kStats) {
    return p.one;
  } else {
    const cchunk_ptr x = (cchunk_ptr)p.chunks + c;
    ChunkDev r;  // field by field: no copy constructor takes a constant-address-space source
    r.k = x->k;
    r.v = x->v;
    r.start = x->start;
    r.len = x->len;
    r.sb = x->sb;
    r.sh = x->sh;
    r.ss = x->ss;
    r.pos0 = x->pos0;
    r.ps = x->ps;
    return r;
  }
}

// ---------------------------------------------------------------------------
// Tile walk (uniform across the workgroup): find the next tile at or after t
// that holds at least one key some query of the workgroup may see.

struct TileInfo {
  int t;           // tile index (== end when the walk is over)
  int cursor;      // chunk containing the tile's first key
  int flags;       // bit 0: all keys from chunk `cursor`; bit 1: the tile runs past the last key
  int kmin, kmax;  // smallest / largest global key position in the tile (causal only)
  int pos0;        // global position of the tile's first row if it lies in one chunk
  int ps;          // position step between rows of chunk `cursor`
  int ss;          // element stride between rows of chunk `cursor`
  int cend;        // index in the concatenation one past the last key of chunk `cursor`
  const char* kp;  // address of the tile's first key row (batch and head applied)
  const char* vp;  // same for values
  int li;          // block-sparse walk: index of the tile in the work item's list
};

// BOUNDS: compute the tile's smallest and largest key position (kmin, kmax)
// over every chunk it touches. Without BOUNDS (the pipelined kernel, whose
// tiles are single increasing position progressions) the causal skip tests
// only the tile's first position, with no loop over chunks: that loop, inlined
// into every step's successor, slowed the whole causal walk by ~9%.
template <int MODE, int ELEM, int TB = BN, bool SKIP = true, bool BOUNDS = true>
__device__ __forceinline__ TileInfo next_tile(const Params& p, int t, int cursor, int end, int qmax, int b,
                                              int hk) {
  TileInfo ti;
  while (t < end) {
    const int64_t t0 = (int64_t)t * TB;
    const int64_t t1 = min(t0 + (int64_t)TB, p.Lk);
    // advance the cursor to the chunk holding key t0 (zero-length chunks are passed over)
    ChunkDev ch = chunk_at<MODE>(p, cursor);
    while (cursor + 1 < p.n_chunks && t0 >= ch.start + ch.len) {
      ++cursor;
      ch = chunk_at<MODE>(p, cursor);
    }
    int kmin = kPosNone, kmax = kPosMin;
    const bool one = (t1 <= ch.start + ch.len);
    if (MODE == kRingCausal && !BOUNDS) {
      if (SKIP && ch.pos0 + ch.ps * (int)(t0 - ch.start) > qmax) {
        // as below: nothing from here to the chunk's end is visible
        const int nt = (int)((ch.start + ch.len) / TB);
        t = nt > t ? nt : t + 1;
        continue;
      }
    } else if (MODE == kRingCausal) {
      int c = cursor;
      ChunkDev cc = ch;
      while (true) {
        const int64_t lo = max(t0, cc.start), hi = min(t1, cc.start + cc.len);
        if (lo < hi) {
          kmin = min(kmin, cc.pos0 + cc.ps * (int)(lo - cc.start));
          kmax = max(kmax, cc.pos0 + cc.ps * (int)(hi - 1 - cc.start));
        }
        if (c + 1 >= p.n_chunks || cc.start + cc.len >= t1) break;
        ++c;
        cc = chunk_at<MODE>(p, c);
      }
      if (SKIP && kmin > qmax) {
        // nothing here is visible, and positions only grow along a chunk, so
        // no later key of chunk `cursor` is visible either: go on at the tile
        // that holds the chunk's end
        const int nt = (int)((ch.start + ch.len) / TB);
        t = nt > t ? nt : t + 1;
        continue;
      }
    }
    const int64_t off = (int64_t)b * ch.sb + (int64_t)hk * ch.sh + (t0 - ch.start) * ch.ss;
    ti.t = t;
    ti.cursor = cursor;
    ti.flags = (one ? 1 : 0) | ((t0 + TB > p.Lk) ? 2 : 0);
    ti.kmin = kmin;
    ti.kmax = kmax;
    ti.pos0 = ch.pos0 + ch.ps * (int)(t0 - ch.start);
    ti.ps = ch.ps;
    ti.ss = (int)ch.ss;
    ti.cend = (int)(ch.start + ch.len);
    ti.kp = (const char*)ch.k + off * ELEM;
    ti.vp = (const char*)ch.v + off * ELEM;
    ti.li = 0;
    return ti;
  }
  ti.li = 0;
  ti.t = end;
  ti.cursor = cursor;
  ti.flags = 1;
  ti.kmin = kPosNone;
  ti.kmax = kPosMin;
  ti.pos0 = 0;
  ti.ps = 1;
  ti.ss = 0;
  ti.cend = 0;
  ti.kp = nullptr;
  ti.vp = nullptr;
  return ti;
}

// The tile after `ti` in the walk. When it lies in the same chunk as `ti` (the
// common case) it follows by scalar arithmetic, with no descriptor load.
template <int MODE, int ELEM, int TB = BN, bool BOUNDS = true>
__device__ __forceinline__ TileInfo successor(const Params& p, const TileInfo& ti, int end, int qmax, int b,
                                              int hk) {
  const int nt = ti.t + 1;
  if (ti.flags == 1 && nt < end && (int64_t)(nt + 1) * TB <= ti.cend &&
      (MODE != kRingCausal || ti.pos0 + TB * ti.ps <= qmax)) {
    TileInfo n = ti;
    n.t = nt;
    n.pos0 = ti.pos0 + TB * ti.ps;
    n.kmin = ti.kmin + TB * ti.ps;
    n.kmax = ti.kmax + TB * ti.ps;
    n.kp = ti.kp + (int64_t)TB * ti.ss * ELEM;
    n.vp = ti.vp + (int64_t)TB * ti.ss * ELEM;
    return n;
  }
  return next_tile<MODE, ELEM, TB, true, BOUNDS>(p, nt, ti.cursor, end, qmax, b, hk);
}

// Reads of tables the kernels never write, through the constant address space:
// a uniform address then becomes a scalar load, which leaves the vector memory
// counter (that the LDS copy pipeline waits on) alone.
typedef const __attribute__((address_space(4))) int* cint_ptr;
typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;
__device__ __forceinline__ int cload(const int* p) { return *(cint_ptr)p; }
__device__ __forceinline__ uint32_t cload(const uint32_t* p) { return *(cu32_ptr)p; }

// Block-sparse walk: the tiles of a work item are entries [first, end) of its
// query tile's list (ascending tile indices). No causal skipping here: the
// list already holds only tiles with a visible pair.
struct SparseWalk {
  const int* list;
  int end;  // one past the work item's last entry
};

// Entries of `list` (n ascending tile indices) below tile t.
__device__ __forceinline__ int lower_entry(const int* list, int n, int t) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cload(list + mid) < t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int MODE, int ELEM, int TB = BN, bool BOUNDS = true>
__device__ __forceinline__ TileInfo sparse_tile(const Params& p, const SparseWalk& sw, int e, int cursor, int end,
                                                int qmax, int b, int hk) {
  if (e >= sw.end) {
    TileInfo ti = next_tile<MODE, ELEM, TB, false, BOUNDS>(p, end, cursor, end, qmax, b, hk);
    ti.li = e;
    return ti;
  }
  TileInfo ti = next_tile<MODE, ELEM, TB, false, BOUNDS>(p, cload(sw.list + e), cursor, end, qmax, b, hk);
  ti.li = e;
  return ti;
}

// The entry after `ti`; a tile right after `ti` in the same chunk follows by
// scalar arithmetic, as in the dense walk.
template <int MODE, int ELEM, int TB = BN, bool BOUNDS = true>
__device__ __forceinline__ TileInfo sparse_successor(const Params& p, const SparseWalk& sw, const TileInfo& ti,
                                                     int end, int qmax, int b, int hk) {
  const int e = ti.li + 1;
  if (e < sw.end) {
    const int nt = cload(sw.list + e);
    if (nt == ti.t + 1 && ti.flags == 1 && (int64_t)(nt + 1) * TB <= ti.cend) {
      TileInfo n = ti;
      n.t = nt;
      n.li = e;
      n.pos0 = ti.pos0 + TB * ti.ps;
      n.kmin = ti.kmin + TB * ti.ps;
      n.kmax = ti.kmax + TB * ti.ps;
      n.kp = ti.kp + (int64_t)TB * ti.ss * ELEM;
      n.vp = ti.vp + (int64_t)TB * ti.ss * ELEM;
      return n;
    }
  }
  return sparse_tile<MODE, ELEM, TB, BOUNDS>(p, sw, e, ti.cursor, end, qmax, b, hk);
}

// Key and value row addresses and position of tile row r; false past the last key.
template <int MODE, int ELEM, int TB = BN>
__device__ __forceinline__ bool row_of(const Params& p, const TileInfo& ti, int r, int b, int hk,
                                       const char*& krow, const char*& vrow, int& pos) {
  const int64_t j = (int64_t)ti.t * TB + r;
  if ((ti.flags & 2) && j >= p.Lk) return false;
  if (ti.flags & 1) {
    krow = ti.kp + (int64_t)r * ti.ss * ELEM;
    vrow = ti.vp + (int64_t)r * ti.ss * ELEM;
    pos = ti.pos0 + r * ti.ps;
    return true;
  }
  int c = ti.cursor;
  ChunkDev ch = chunk_at<MODE>(p, c);
  while (c + 1 < p.n_chunks && j >= ch.start + ch.len) {
    ++c;
    ch = chunk_at<MODE>(p, c);
  }
  const int64_t off = (int64_t)b * ch.sb + (int64_t)hk * ch.sh + (j - ch.start) * ch.ss;
  krow = (const char*)ch.k + off * ELEM;
  vrow = (const char*)ch.v + off * ELEM;
  pos = ch.pos0 + ch.ps * (int)(j - ch.start);
  return true;
}

// True when every row of the tile comes from one chunk, none lies past the last
// key, and rows are 16-byte aligned runs of exactly `dp` elements: then the
// tile can be fetched with unconditional vector loads (a uniform condition).
__device__ __forceinline__ bool fast_tile(const Params& p, const TileInfo& ti, int dp) {
  return ti.flags == 1 && p.vec && p.d == dp;
}

// ---------------------------------------------------------------------------
// Element-type specific pieces: LDS layout, tile staging, MFMA fragments.

template <class T, int DP>
struct Ops;

// bf16: K row-major [BN][DP + 8]; V transposed [DP][BN + 8] with the key order of
// each 16-key slice permuted (quads 1 and 2 swapped) to match the P fragments,
// followed by the BN key positions of the tile.
template <int DP>
struct Ops<__bf16, DP> {
  static constexpr int KP = DP + 8;
  static constexpr int VP = BN + 8;
  static constexpr int K_BYTES = BN * KP * 2;
  static constexpr int V_BYTES = DP * VP * 2 + BN * 4;
  static constexpr int POS_OFF = DP * VP * 2;
  static constexpr int CPR = DP / 8;                                     // 16-byte chunks per row
  static constexpr int NK = (BN * CPR + kThreads - 1) / kThreads;        // K items per thread
  static constexpr int NV = ((BN / 4) * CPR + kThreads - 1) / kThreads;  // V quad items per thread
  static constexpr int QF = DP / 16;

  struct StageK {
    u32x4 k[NK];
  };
  struct StageV {
    u32x4 v[NV][4];
    int pos[NV][4];
  };
  struct QFrag {
    bf16x8 f[QF];
  };

  static __device__ __forceinline__ u32x4 load16(const __bf16* row, int c0, int d, bool vec) {
    if (vec) {
      if (c0 < d) return gload16(row + c0);
      return u32x4{0, 0, 0, 0};
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = (c0 + 2 * i < d) ? gload_u16(row + c0 + 2 * i) : 0u;
      uint32_t hi = (c0 + 2 * i + 1 < d) ? gload_u16(row + c0 + 2 * i + 1) : 0u;
      w[i] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }

  static __device__ __forceinline__ void load_q(const Params& p, const __bf16* qrow, bool valid, int h,
                                                QFrag& q) {
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      u32x4 x = valid ? load16(qrow, kk * 16 + h * 8, p.d, p.vec) : u32x4{0, 0, 0, 0};
      q.f[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Raw scores <q, k> of the tile, transposed: s[kb][r] is key kb*32 + 8(r/4) + 4h + r%4.
  static __device__ __forceinline__ void qk(const char* kbuf, const QFrag& q, f32x16* s, int lane) {
    const __bf16* base = (const __bf16*)kbuf + (lane & 31) * KP + (lane >> 5) * 8;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        bf16x8 a = *(const bf16x8*)(base + kb * 32 * KP + kk * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.f[kk], s[kb], 0, 0, 0);
      }
    }
  }

  // o[db] += V^T P^T over the tile, P taken from the exponentiated score blocks.
  static __device__ __forceinline__ void pv(const char* vbuf, const f32x16* s, f32x16* o, int lane) {
    const __bf16* Vs = (const __bf16*)vbuf;
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int t = 0; t < 8; ++t) pf[ks][t] = (__bf16)s[ks >> 1][(ks & 1) * 8 + t];
    }
    const __bf16* vrow = Vs + (lane & 31) * VP + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) {
        bf16x8 a = *(const bf16x8*)(vrow + db * 32 * VP + ks * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ void fetch_k(const Params& p, const TileInfo& ti, int b, int hk, int tid,
                                                 StageK& st) {
    if (fast_tile(p, ti, DP)) {
      // one chunk, no tail, aligned rows of exactly DP elements: straight-line loads
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int item = tid + i * kThreads;
        if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
          const int r = item / CPR, cc = item % CPR;
          st.k[i] = gload16(ti.kp + ((int64_t)r * ti.ss + cc * 8) * 2);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      st.k[i] = u32x4{0, 0, 0, 0};
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        const char *kr, *vr;
        int pos;
        if (row_of<MODE, 2>(p, ti, r, b, hk, kr, vr, pos)) st.k[i] = load16((const __bf16*)kr, cc * 8, p.d, p.vec);
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ void fetch_v(const Params& p, const TileInfo& ti, int b, int hk, int tid,
                                                 StageV& st) {
    if (fast_tile(p, ti, DP)) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int item = tid + i * kThreads;
        if (((BN / 4) * CPR) % kThreads == 0 || item < (BN / 4) * CPR) {
          const int qd = item % (BN / 4), cc = item / (BN / 4);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            st.v[i][w] = gload16(ti.vp + ((int64_t)(qd * 4 + w) * ti.ss + cc * 8) * 2);
            st.pos[i][w] = ti.pos0 + (qd * 4 + w) * ti.ps;
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int item = tid + i * kThreads;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        st.v[i][w] = u32x4{0, 0, 0, 0};
        st.pos[i][w] = kPosNone;
      }
      if (((BN / 4) * CPR) % kThreads == 0 || item < (BN / 4) * CPR) {
        const int qd = item % (BN / 4), cc = item / (BN / 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const char *kr, *vr;
          int pos;
          if (row_of<MODE, 2>(p, ti, qd * 4 + w, b, hk, kr, vr, pos)) {
            st.v[i][w] = load16((const __bf16*)vr, cc * 8, p.d, p.vec);
            st.pos[i][w] = pos;
          }
        }
      }
    }
  }

  static __device__ __forceinline__ void store_k(char* kbuf, const StageK& st, int tid) {
    __bf16* Ks = (__bf16*)kbuf;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        *(u32x4*)(Ks + r * KP + cc * 8) = st.k[i];
      }
    }
  }

  static __device__ __forceinline__ void store_v(char* vbuf, const StageV& st, int tid) {
    __bf16* Vs = (__bf16*)vbuf;
    int* P = (int*)(vbuf + POS_OFF);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int item = tid + i * kThreads;
      if (((BN / 4) * CPR) % kThreads == 0 || item < (BN / 4) * CPR) {
        const int qd = item % (BN / 4), cc = item / (BN / 4);
        const int qi = qd & 3;
        const int pq = (qd & ~3) | (qi == 1 ? 2 : (qi == 2 ? 1 : qi));
        const u32x4* r = st.v[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dword w of each key row holds d = 2w (low half) and d = 2w + 1 (high half)
          const uint32_t e0 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
          const uint32_t e1 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
          const uint32_t o0 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
          const uint32_t o1 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
          *(u32x2*)(Vs + (cc * 8 + 2 * w) * VP + pq * 4) = u32x2{e0, e1};
          *(u32x2*)(Vs + (cc * 8 + 2 * w + 1) * VP + pq * 4) = u32x2{o0, o1};
        }
        if (cc == 0) {
#pragma unroll
          for (int w = 0; w < 4; ++w) P[qd * 4 + w] = st.pos[i][w];
        }
      }
    }
  }
};

// fp32: K and V both row-major [BN][DP + 4] (V followed by the key positions);
// fragments for v_mfma_f32_32x32x2f32.
template <int DP>
struct Ops<float, DP> {
  static constexpr int KP = DP + 4;
  static constexpr int K_BYTES = BN * KP * 4;
  static constexpr int V_BYTES = BN * KP * 4 + BN * 4;
  static constexpr int POS_OFF = BN * KP * 4;
  static constexpr int CPR = DP / 4;
  static constexpr int NK = (BN * CPR + kThreads - 1) / kThreads;
  static constexpr int QF = DP / 2;

  struct StageK {
    u32x4 k[NK];
  };
  struct StageV {
    u32x4 v[NK];
    int pos[NK];
  };
  struct QFrag {
    float f[QF];
  };

  static __device__ __forceinline__ u32x4 load16(const float* row, int c0, int d, bool vec) {
    if (vec) {
      if (c0 < d) return gload16(row + c0);
      return u32x4{0, 0, 0, 0};
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (c0 + i < d) ? __float_as_uint(gload_f32(row + c0 + i)) : 0u;
    return u32x4{w[0], w[1], w[2], w[3]};
  }

  static __device__ __forceinline__ void load_q(const Params& p, const float* qrow, bool valid, int h,
                                                QFrag& q) {
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      const int c = 2 * kk + h;
      q.f[kk] = (valid && c < p.d) ? gload_f32(qrow + c) : 0.f;
    }
  }

  static __device__ __forceinline__ void qk(const char* kbuf, const QFrag& q, f32x16* s, int lane) {
    const float* base = (const float*)kbuf + (lane & 31) * KP + (lane >> 5);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < QF; ++kk)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(base[kb * 32 * KP + 2 * kk], q.f[kk], s[kb], 0, 0, 0);
    }
  }

  static __device__ __forceinline__ void pv(const char* vbuf, const f32x16* s, f32x16* o, int lane) {
    const float* Vs = (const float*)vbuf;
    const int h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < DP / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * KP + db * 32 + (lane & 31)], s[kb][r], o[db], 0,
                                                       0, 0);
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ void fetch_k(const Params& p, const TileInfo& ti, int b, int hk, int tid,
                                                 StageK& st) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      st.k[i] = u32x4{0, 0, 0, 0};
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        const char *kr, *vr;
        int pos;
        if (row_of<MODE, 4>(p, ti, r, b, hk, kr, vr, pos)) st.k[i] = load16((const float*)kr, cc * 4, p.d, p.vec);
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ void fetch_v(const Params& p, const TileInfo& ti, int b, int hk, int tid,
                                                 StageV& st) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      st.v[i] = u32x4{0, 0, 0, 0};
      st.pos[i] = kPosNone;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        const char *kr, *vr;
        int pos;
        if (row_of<MODE, 4>(p, ti, r, b, hk, kr, vr, pos)) {
          st.v[i] = load16((const float*)vr, cc * 4, p.d, p.vec);
          st.pos[i] = pos;
        }
      }
    }
  }

  static __device__ __forceinline__ void store_k(char* kbuf, const StageK& st, int tid) {
    float* Ks = (float*)kbuf;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        *(u32x4*)(Ks + r * KP + cc * 4) = st.k[i];
      }
    }
  }

  static __device__ __forceinline__ void store_v(char* vbuf, const StageV& st, int tid) {
    float* Vs = (float*)vbuf;
    int* P = (int*)(vbuf + POS_OFF);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int item = tid + i * kThreads;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        const int r = item / CPR, cc = item % CPR;
        *(u32x4*)(Vs + r * KP + cc * 4) = st.v[i];
        if (cc == 0) P[r] = st.pos[i];
      }
    }
  }
};

// ---------------------------------------------------------------------------

__device__ __forceinline__ int query_pos(const Params& p, int64_t row) {
  for (int s = 0; s < p.n_qseg; ++s) {
    QSegDev g = p.qsegs[s];
    if (row < g.row0 + g.len) return (int)(g.pos0 + g.ps * (row - g.row0));
  }
  return kPosMin;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Per-wave view of a tile: 0 = nothing visible, 1 = everything visible, 2 = mixed.
__device__ __forceinline__ int wave_mode(const TileInfo& ti, int wqmin, int wqmax, bool causal) {
  if (causal) {
    if (ti.kmin > wqmax) return 0;
    if ((ti.flags & 2) || ti.kmax > wqmin) return 2;
    return 1;
  }
  return (ti.flags & 2) ? 2 : 1;
}

// Work item of a workgroup and the query row of each lane.
struct Work {
  int b, hk, hq, split;
  int qt;                   // query tile (rows qt * rows per workgroup onwards)
  int64_t qrow_idx;         // (batch, head, row) index of the lane's query row
  bool valid;               // the lane's row exists
  int qpos;                 // global position of the lane's query (causal), else kPosAll
  int spos;                 // global position of the lane's query (block-sparse calls), else 0
  int wqmin, wqmax, gqmax;  // bounds of the query positions over the wave and the workgroup
};

template <int MODE, int W = kWaves, bool SP = false>
__device__ __forceinline__ Work decode_work(const Params& p, int* qred, int wave, int lane) {
  Work wk;
  // Blocks are dealt to the 8 XCDs round-robin; remap so that each XCD gets a
  // contiguous range of work items, and order items so that the blocks sharing
  // one key/value head and key range (all query tiles of a head, and all query
  // heads of a GQA group) are adjacent and share that XCD's L2.
  int w = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) w = (w & 7) * (nwg >> 3) + (w >> 3);
  const int group = p.Hq / p.Hkv;
  const int g = w % group;
  w /= group;
  int qt = w % p.n_qt;
  w /= p.n_qt;
  wk.split = w % p.nsplit;
  w /= p.nsplit;
  wk.hk = w % p.Hkv;
  wk.b = w / p.Hkv;
  if (MODE == kRingCausal) qt = p.n_qt - 1 - qt;  // later queries see more keys: start them first
  wk.hq = wk.hk * group + g;

  wk.qt = qt;
  const int64_t row = (int64_t)qt * (32 * W) + wave * 32 + (lane & 31);
  wk.valid = row < p.Lq;
  wk.qrow_idx = ((int64_t)wk.b * p.Hq + wk.hq) * p.Lq + (wk.valid ? row : 0);
  wk.spos = (SP && wk.valid) ? query_pos(p, row) : 0;

  wk.qpos = kPosAll;
  wk.wqmin = kPosAll;
  wk.wqmax = kPosAll;
  wk.gqmax = kPosAll;
  if (MODE == kRingCausal) {
    wk.qpos = wk.valid ? query_pos(p, row) : kPosMin;
    wk.wqmin = __builtin_amdgcn_readfirstlane(wave_min(wk.valid ? wk.qpos : kPosNone));
    wk.wqmax = __builtin_amdgcn_readfirstlane(wave_max(wk.valid ? wk.qpos : kPosMin));
    if (lane == 0) {
      qred[wave] = wk.wqmin;
      qred[W + wave] = wk.wqmax;
    }
    __syncthreads();
    int gq = qred[W];
#pragma unroll
    for (int i = 1; i < W; ++i) gq = max(gq, qred[W + i]);
    wk.gqmax = __builtin_amdgcn_readfirstlane(gq);
  }
  return wk;
}

// Epilogue: combine the two half-waves' denominators, then write the lane's row
// (normalised output and lse, chunk statistics, or a key-range partial).
template <int DP, int MODE>
__device__ __forceinline__ void write_rows(const Params& p, const Work& wk, f32x16* o, float l_run, float m_ref,
                                           float m_max, int h) {
  float l = sum_xor32(l_run);
  if (MODE == kStats && m_max != m_ref) {
    // report statistics relative to the true row maximum
    const float f = __builtin_amdgcn_exp2f((m_ref - m_max) * p.c2);
    l *= f;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) o[db] *= f;
    m_ref = m_max;
  }
  if (!wk.valid) return;
  float* orow;
  float inv = 1.f;
  if (p.nsplit > 1) {
    const int64_t rows = (int64_t)p.B * p.Hq * p.Lq;
    orow = p.part + ((int64_t)wk.split * rows + wk.qrow_idx) * p.d;
  } else {
    orow = p.o + wk.qrow_idx * p.d;
    if (MODE != kStats) inv = (l > 0.f) ? 1.f / l : 0.f;
  }
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int c0 = db * 32 + 8 * gi + 4 * h;
      const f32x4 v = {o[db][4 * gi] * inv, o[db][4 * gi + 1] * inv, o[db][4 * gi + 2] * inv,
                       o[db][4 * gi + 3] * inv};
      if (c0 + 3 < p.d && (p.d & 3) == 0) {
        *(f32x4*)(orow + c0) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + i < p.d) orow[c0 + i] = v[i];
      }
    }
  }
  if (h == 0) {
    if (p.nsplit > 1) {
      const int64_t rows = (int64_t)p.B * p.Hq * p.Lq;
      float* pl = p.part + (int64_t)p.nsplit * rows * p.d;
      pl[(int64_t)wk.split * rows + wk.qrow_idx] = l;
      pl[((int64_t)p.nsplit + wk.split) * rows + wk.qrow_idx] = m_ref;  // raw units
    } else {
      const float m_out = (m_ref == -INFINITY) ? -INFINITY : m_ref * p.scale;
      if (MODE == kStats) {
        p.l[wk.qrow_idx] = l;
        p.m[wk.qrow_idx] = m_out;
      } else if (p.l != nullptr) {
        p.l[wk.qrow_idx] = (l > 0.f) ? m_out + logf(l) : -INFINITY;
      }
    }
  }
}

// Tile walk state with every field forced into scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ TileInfo uniform(TileInfo t) {
  t.t = __builtin_amdgcn_readfirstlane(t.t);
  t.cursor = __builtin_amdgcn_readfirstlane(t.cursor);
  t.flags = __builtin_amdgcn_readfirstlane(t.flags);
  t.kmin = __builtin_amdgcn_readfirstlane(t.kmin);
  t.kmax = __builtin_amdgcn_readfirstlane(t.kmax);
  t.pos0 = __builtin_amdgcn_readfirstlane(t.pos0);
  t.ps = __builtin_amdgcn_readfirstlane(t.ps);
  t.ss = __builtin_amdgcn_readfirstlane(t.ss);
  t.cend = __builtin_amdgcn_readfirstlane(t.cend);
  t.kp = uniform_ptr(t.kp);
  t.vp = uniform_ptr(t.vp);
  t.li = __builtin_amdgcn_readfirstlane(t.li);
  return t;
}

// fp32 kernel: one tile per iteration, K and V of the next tile fetched from
// HBM into registers while the current tile is computed.
// With SP (block-sparse calls) the tiles come from the work item's list and
// every score of a visited tile is checked against the block mask as well.
template <class T, int DP, int MODE, bool SP = false>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(Params p) {
  using O = Ops<T, DP>;
  __shared__ __attribute__((aligned(16))) char kbuf[2][O::K_BYTES];
  __shared__ __attribute__((aligned(16))) char vbuf[2][O::V_BYTES];
  __shared__ int qred[2 * kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;

  const Work wk = decode_work<MODE, kWaves, SP>(p, qred, wave, lane);
  const int b = wk.b, hk = wk.hk, split = wk.split;
  const bool valid = wk.valid;
  const int64_t qrow_idx = wk.qrow_idx;
  const int qpos = wk.qpos, wqmin = wk.wqmin, wqmax = wk.wqmax, gqmax = wk.gqmax;

  typename O::QFrag qf;
  O::load_q(p, (const T*)p.q + qrow_idx * p.d, valid, h, qf);
  // Drain the query loads here, once: otherwise the wait-count analysis carries
  // them into the tile loop and drains every HBM prefetch at each tile.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  f32x16 o[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max (raw dot products <q, k>) that u and l are relative to
  float m_max = -INFINITY;  // true running max (the chunk-stats call reports it)
  float l_run = 0.f;        // this lane's share of the running denominator

  // This workgroup's key tiles: range `split` of nsplit equal ranges.
  const int ntiles = (int)((p.Lk + BN - 1) / BN);
  const int tbeg = (int)((int64_t)ntiles * split / p.nsplit);
  const int tend = (int)((int64_t)ntiles * (split + 1) / p.nsplit);
  constexpr int ELEM = sizeof(T);

  typename O::StageK sk;
  typename O::StageV sv;
  f32x16 s0[BN / 32];

  // Softmax of one tile (its raw scores in s), folded into the running state,
  // then O += P V with the tile's V from LDS.
  auto consume = [&](f32x16* s, int mode, const char* vb_) {
    if (mode == 2) {
      const int* kp = (const int*)(vb_ + O::POS_OFF);
#pragma unroll
      for (int k2 = 0; k2 < BN / 32; ++k2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k2 * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kp[key] > qpos) s[k2][r] = -INFINITY;
        }
      if constexpr (SP) {
        // block mask: the lane's query block row, one bit per key block
        const uint32_t* row = p.sp_bits + (int64_t)(wk.spos >> p.sp_lgq) * p.sp_rw;
#pragma unroll
        for (int k2 = 0; k2 < BN / 32; ++k2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kpos = kp[k2 * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
            if (kpos != kPosNone) {
              const int kb = kpos >> p.sp_lgk;
              if (!((row[kb >> 5] >> (kb & 31)) & 1u)) s[k2][r] = -INFINITY;
            }
          }
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < BN / 32; ++k2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mt = fmax_raw(mt, fmax_raw(s[k2][r], s[k2][r + 1]));
    mt = max_xor32(mt);
    if constexpr (MODE == kStats) m_max = fmax_raw(m_max, mt);
    // move the reference when a score exceeds it by more than 2^kLazy
    const bool need = mt * p.c2 > m_ref * p.c2 + kLazy;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f((m_ref - mt) * p.c2) : 1.f;
      if (need) m_ref = mt;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) o[db] *= alpha;
    }
    const float ms = (m_ref == -INFINITY) ? 0.f : m_ref * p.c2;
    float rs = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < BN / 32; ++k2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[k2][r], p.c2, -ms));
        s[k2][r] = e;
        rs += e;
      }
    l_run += rs;
    __builtin_amdgcn_s_setprio(1);
    O::pv(vb_, s, o, lane);
    __builtin_amdgcn_s_setprio(0);
  };

  // K and V of a tile are staged together; the tile after is fetched from HBM
  // into registers while this one is computed.
  SparseWalk sw = {nullptr, 0};
  int e0 = 0;
  if constexpr (SP) {
    sw.list = p.sp_list + (int64_t)wk.qt * p.sp_cap;
    const int cnt = p.sp_count[wk.qt];
    e0 = lower_entry(sw.list, cnt, tbeg);
    sw.end = lower_entry(sw.list, cnt, tend);
  }
  TileInfo cur = SP ? sparse_tile<MODE, ELEM>(p, sw, e0, 0, tend, gqmax, b, hk)
                    : next_tile<MODE, ELEM>(p, tbeg, 0, tend, gqmax, b, hk);
  if (cur.t < tend) {
    O::template fetch_k<MODE>(p, cur, b, hk, tid, sk);
    O::template fetch_v<MODE>(p, cur, b, hk, tid, sv);
    O::store_k(kbuf[0], sk, tid);
    O::store_v(vbuf[0], sv, tid);
  }
  int bi = 0;
  while (cur.t < tend) {
    const TileInfo nxt = SP ? sparse_successor<MODE, ELEM>(p, sw, cur, tend, gqmax, b, hk)
                            : successor<MODE, ELEM>(p, cur, tend, gqmax, b, hk);
    if (nxt.t < tend) {
      O::template fetch_k<MODE>(p, nxt, b, hk, tid, sk);
      O::template fetch_v<MODE>(p, nxt, b, hk, tid, sv);
    }
    __syncthreads();  // K(cur) and V(cur) are in LDS
    int mode = wave_mode(cur, wqmin, wqmax, MODE == kRingCausal);
    if (SP && mode == 1) mode = 2;  // the block mask is checked per score
    if (mode) {
      // Raised priority while issuing matrix ops: of the two waves sharing a
      // SIMD, the one with MFMAs ready goes first and the other fills VALU slots.
      __builtin_amdgcn_s_setprio(1);
      O::qk(kbuf[bi], qf, s0, lane);
      __builtin_amdgcn_s_setprio(0);
      consume(s0, mode, vbuf[bi]);
    }
    if (nxt.t < tend) {
      O::store_k(kbuf[bi ^ 1], sk, tid);
      O::store_v(vbuf[bi ^ 1], sv, tid);
    }
    bi ^= 1;
    cur = nxt;
  }

  write_rows<DP, MODE>(p, wk, o, l_run, m_ref, m_max, h);
}

// Pipelined bf16 path. K and V tiles are row-major [BN][DP] without padding,
// the 16-byte pieces of each row permuted by an XOR swizzle (piece c of row r
// sits at position c ^ swz(r)) so that the MFMA operand reads hit distinct LDS
// banks.
//
// Tiles are copied from HBM straight into LDS (global_load_lds, 16 bytes per
// lane: the lanes of a wave fill 1 KB of consecutive LDS, and each lane loads
// the piece that belongs in its slot). Slots that hold no data (rows past the
// last key, pieces past head_dim) load a valid piece of the same tile instead:
// such keys are masked and such columns meet zero query columns or are never
// written out, so any finite value will do.
//
// Operand reads: the K operand of S^T = K Q^T is one ds_read_b128 per MFMA;
// the V^T operand of O^T = V^T P^T is two ds_read_b64_tr_b16 per MFMA, which
// transpose 4x4 blocks of 16-bit values across each group of 16 lanes (lane i
// of a group receives element i % 4 of source lanes 4k + i / 4, k = 0..3).
template <int DP, int TB, int NT>
struct PipeOps {
  static constexpr int CPR = DP / 8;                // 16-byte pieces per row
  static constexpr int ROWB = DP * 2;               // bytes per row
  static constexpr int TILE_B = TB * ROWB;          // bytes of a K or V tile
  static constexpr int NS = TB * CPR / NT;    // 16-byte pieces per thread and tile
  static constexpr int QF = DP / 16;
  static_assert(NS * NT == TB * CPR, "whole pieces per thread");

  // Swizzle: distinct banks for 16 consecutive rows at one piece (K reads) and
  // for 4 consecutive rows x 4 consecutive pieces (transposing V reads).
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (DP == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (DP == 64) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }

  struct QFrag {
    bf16x8 f[QF];
  };
  // Per-lane LDS byte offsets of the MFMA operands, fixed for the whole kernel.
  struct Lanes {
    int k[QF];          // K operand of k-step kk (add kb * 32 rows)
    int v[DP / 32][2];  // V operand of d-block db, half h (add ks * 16 rows)
  };

  static __device__ __forceinline__ Lanes lanes(int lane) {
    Lanes L;
    const int r = lane & 31, hsel = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) L.k[kk] = r * ROWB + (((2 * kk + hsel) ^ swz(r)) << 4);
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // rows: keys 4(g/2) + 8hh + j/4 of the 16-key slice; 4 d values from 32db + 16(g%2) + 4(j%4)
        const int row = 4 * (g >> 1) + 8 * hh + (j >> 2);
        const int d0 = 32 * db + 16 * (g & 1) + 4 * (j & 3);
        L.v[db][hh] = row * ROWB + (((d0 >> 3) ^ swz(row)) << 4) + 2 * (d0 & 7);
      }
    return L;
  }

  static __device__ __forceinline__ u32x4 load16(const __bf16* row, int c0, int d, bool vec) {
    if (vec) {
      if (c0 < d) return gload16(row + c0);
      return u32x4{0, 0, 0, 0};
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = (c0 + 2 * i < d) ? gload_u16(row + c0 + 2 * i) : 0u;
      uint32_t hi = (c0 + 2 * i + 1 < d) ? gload_u16(row + c0 + 2 * i + 1) : 0u;
      w[i] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }

  static __device__ __forceinline__ void load_q(const Params& p, const __bf16* qrow, bool valid, int h,
                                                QFrag& q) {
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      u32x4 x = valid ? load16(qrow, kk * 16 + h * 8, p.d, p.vec) : u32x4{0, 0, 0, 0};
      q.f[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Raw scores <q, k> of the tile, transposed: s[kb][r] is key kb*32 + 8(r/4) + 4h + r%4.
  static __device__ __forceinline__ void qk(const char* kbuf, const QFrag& q, const Lanes& L, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < TB / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
#pragma unroll
      for (int kb = 0; kb < TB / 32; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kbuf + L.k[kk] + kb * 32 * ROWB);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.f[kk], s[kb], 0, 0, 0);
      }
    }
  }

  // Slot s = i * NT + tid of a tile holds physical piece s % CPR of row
  // s / CPR. Byte offset, from the tile's first row, of the piece that slot i
  // of this thread receives in a tile of row stride ss2 bytes.
  static __device__ __forceinline__ uint32_t piece_offset(int i, int tid, uint32_t ss2) {
    const int sl = i * NT + tid;
    const int r = sl / CPR, c = (sl % CPR) ^ swz(r);
    return (uint32_t)r * ss2 + (uint32_t)(c * 16);
  }

  // The copies are issued from inline assembly. The compiler's wait-count
  // analysis, when it sees LDS written by global_load_lds, waits for every
  // outstanding LDS read before each use of one (lgkmcnt(0)), which exposes the
  // LDS latency at every MFMA. Here the copies are invisible to it; the kernel
  // waits for them itself (vmcnt) before the barrier that publishes a tile.
  static __device__ __forceinline__ uint32_t lds_addr(char* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) char*)p);
  }
  static __device__ __forceinline__ void copy16(const char* src, char* dst_wave) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_addr(dst_wave))
                 : "memory", "m0");
  }
  static __device__ __forceinline__ void copy16_base(const char* base, uint32_t off, char* dst_wave) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds_addr(dst_wave))
                 : "memory", "m0");
  }

  // Tile in one chunk, no tail, head_dim == DP: uniform base plus 32-bit lane offsets.
  static __device__ __forceinline__ void copy_fast(const char* base, const uint32_t* off, char* dst, int wave) {
#pragma unroll
    for (int i = 0; i < NS; ++i) copy16_base(base, off[i], dst + (i * NT + wave * 64) * 16);
  }

  // Any other tile: each slot's row is looked up chunk by chunk.
  template <int MODE>
  static __device__ __forceinline__ void copy_slow(const Params& p, const TileInfo& ti, int b, int hk, int tid,
                                                   int wave, bool is_v, char* dst) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int sl = i * NT + tid;
      const int r = sl / CPR;
      int c = (sl % CPR) ^ swz(r);
      const char *kr, *vr;
      int pos;
      if (!row_of<MODE, 2, TB>(p, ti, r, b, hk, kr, vr, pos)) row_of<MODE, 2, TB>(p, ti, 0, b, hk, kr, vr, pos);
      if (c * 8 >= p.d) c = 0;
      copy16((is_v ? vr : kr) + c * 16, dst + (i * NT + wave * 64) * 16);
    }
  }
};

// ---------------------------------------------------------------------------
// bf16 kernel, software-pipelined inside each wave. Iteration j computes the
// scores of tile j+1 on the matrix cores while the vector ALUs exponentiate
// tile j and the matrix cores accumulate P(j) V(j): one phase of fixed slots,
// each holding one score MFMA, one output MFMA and a share of the vector work
// (see `fused`). A wave's own vector instructions issued between its MFMAs run
// while the matrix core works; spreading them evenly keeps both busy. The row
// maximum of tile j+1 is taken in the last slots, from score blocks finished
// earlier in the phase, so no vector instruction waits on an MFMA in flight.
//
// LDS holds a ring of NB K buffers and NB V buffers: iteration j reads K(j+1)
// and V(j) and fills K(j+1+D) and V(j+D), straight from HBM, into buffers read
// D iterations earlier; one barrier per iteration.

template <int N>
struct IntC {
  static constexpr int value = N;
};

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations and nothing else (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// Causal masks (and the ragged last tile) use the fact that on this path the
// keys of a tile have positions pos0 + kps * key in one arithmetic progression
// (kps = 1 for contiguous shards): key `key` is masked for the lane's query
// when key > min(floor((qpos - pos0) / kps), keys in the tile - 1). MASK
// selects the variant that applies it to every tile (1: kps = 1; 2: any kps,
// at the cost of an fp64 multiply per lane and step); with MASK = 0 no
// tile needs one (no causal mask and a whole number of tiles).
//
// SP (block-sparse calls, MASK = 1): the tiles come from the work item's list,
// and every row of a wave lies in one query block while a tile spans at most
// two key blocks, so the block mask admits one run [lo, hi] of each tile's keys
// per wave; lo joins the per-lane upper bound above.
template <int DP, int MODE, int MASK, bool SP = false>
__global__ __launch_bounds__(64 * pipe_waves(MODE), pipe_resident(MODE)) void attention_bf16_kernel(Params p) {
  constexpr int W = pipe_waves(MODE);
  constexpr int kPipeThreads = 64 * W;
  constexpr int kPipeResident = pipe_resident(MODE);
  constexpr int TB = pipe_tile(DP);
  using O = PipeOps<DP, TB, kPipeThreads>;
  constexpr int NM = DP * TB / 512;  // score (and output) MFMAs per tile and wave
  constexpr int QF_ = O::QF;
  // Buffers per LDS ring (the resident workgroups of a CU share 160 KB) and
  // tiles copied ahead of the one being read.
  constexpr int NB = 2 * O::TILE_B * 4 * kPipeResident <= 160 * 1024 ? 4 : 2;
  constexpr int D = NB - 1;
  // One array per ring slot: copies into one slot and reads of another are
  // then provably disjoint, and the compiler does not make the reads wait for
  // the copies (it inserts those waits when it cannot tell them apart).
  static_assert(NB == 2 || NB == 4, "two or four slots per ring");
  constexpr int XB = NB == 4 ? O::TILE_B : 16;  // size of slots 2 and 3
  __shared__ __attribute__((aligned(16))) char k0[O::TILE_B], k1[O::TILE_B], k2[XB], k3[XB];
  __shared__ __attribute__((aligned(16))) char v0[O::TILE_B], v1[O::TILE_B], v2[XB], v3[XB];
  char* const kbuf[4] = {k0, k1, k2, k3};
  char* const vbuf[4] = {v0, v1, v2, v3};
  __shared__ int qred[2 * W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;

  const Work wk = decode_work<MODE, W, SP>(p, qred, wave, lane);
  const int b = wk.b, hk = wk.hk;
  const typename O::Lanes L = O::lanes(lane);
  // block-sparse calls: the wave's query block (the same for all its rows)
  const int wqb = SP ? __builtin_amdgcn_readfirstlane(wk.valid ? wk.spos >> p.sp_lgq : 0) : 0;

  typename O::QFrag qf;
  O::load_q(p, (const __bf16*)p.q + wk.qrow_idx * p.d, wk.valid, h, qf);
  // Drain the query loads here, once: otherwise the wait-count analysis carries
  // them into the tile loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  f32x16 o[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max (raw dot products <q, k>) that u and l are relative to
  float m_max = -INFINITY;  // true running max (the chunk-stats call reports it)
  float l_run = 0.f;        // this lane's share of the running denominator
  float alpha = 1.f;        // factor taking l and u to the reference of the next tile to exponentiate
  float ms = 0.f;           // that reference, in exp2 units
  bool rescale = false;     // some lane of the wave has alpha != 1
  const float c2 = p.c2;

  const int ntiles = (int)((p.Lk + TB - 1) / TB);
  const int tbeg = (int)((int64_t)ntiles * wk.split / p.nsplit);
  const int tend = (int)((int64_t)ntiles * (wk.split + 1) / p.nsplit);

  // Row maximum of a tile's scores (already masked), in two parts: this lane's
  // share, then the merge over the two lanes of the row and the reference
  // update. The reference moves when a score exceeds it by more than 2^kLazy.
  // A tile that does not exist (real == false) leaves the state unchanged.
  auto lane_max = [&](const f32x16* s) {
    float mt = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < TB / 32; ++k2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mt = fmax_raw(mt, fmax_raw(s[k2][r], s[k2][r + 1]));
    return mt;
  };
  auto finish_max = [&](float mt, bool real) {
    mt = max_xor32(mt);
    if constexpr (MODE == kStats) m_max = real ? fmax_raw(m_max, mt) : m_max;
    const bool need = real && mt * c2 > m_ref * c2 + kLazy;
    alpha = need ? __builtin_amdgcn_exp2f((m_ref - mt) * c2) : 1.f;
    m_ref = need ? mt : m_ref;
    ms = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    rescale = __any(need);
  };

  auto rescale_o = [&]() {
    if (rescale) {
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) o[db] *= alpha;
    }
  };

  // One iteration's matrix work, in NM + NDB slots of fixed content. Slot i
  // issues score MFMA i of S(j+1) (i < NM) and output MFMA i - NDB of
  // O += P(j) V(j) (i >= NDB); it exponentiates the share of P(j) that the
  // output MFMAs of slot i + NDB consume, takes lane maxima of score blocks
  // that earlier slots finished, and issues the LDS reads of slot i + kRA.
  // Scheduling barriers split every slot in two, each half one MFMA and part
  // of the slot's vector work, so the vector work runs under the MFMAs and
  // neither MFMA waits on the other with nothing behind it. Score MFMAs go
  // k-step-major over groups of two blocks, which finishes the first group
  // half way through.
  constexpr int NBK = TB / 32;         // score blocks of 32 keys
  constexpr int NDB = DP / 32;         // output blocks of 32 columns
  constexpr int NSL = NM + NDB;        // slots
  constexpr int GB = NBK >= 2 ? 2 : 1; // score blocks per group
  constexpr int NG = NBK / GB;         // groups
  constexpr int VPS = 8 / NDB;         // P values per slot (8 per 16-key step)
  constexpr int kRA = 2;               // slots between an LDS read and its use
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
  auto fused = [&](const char* __restrict__ k_read, const char* __restrict__ v_read, const f32x16* sc, f32x16* sn,
                   float& mt_out) {
    bf16x8 ka[NSL], va[NSL];
    uint32_t pw[TB / 16][4];
    auto read_slot = [&](int sl) {
      if (sl < NM) {
        const int g = sl / (QF_ * GB), kk = (sl % (QF_ * GB)) / GB, kb = g * GB + sl % GB;
        ka[sl] = *(const bf16x8*)(k_read + L.k[kk] + kb * 32 * O::ROWB);
      }
      const int pi = sl - NDB;
      if (pi >= 0) {
        const int ks = pi / NDB, db = pi % NDB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(v_read + L.v[db][0] + ks * 16 * O::ROWB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(v_read + L.v[db][1] + ks * 16 * O::ROWB));
        va[sl] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    float rs0 = 0.f, rs1 = 0.f;
    float mx[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) mx[g][0] = mx[g][1] = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < kRA; ++sl) read_slot(sl);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl + kRA < NSL) read_slot(sl + kRA);
      // First half of the slot: the score MFMA and the first half of the
      // exponentials; second half: the output MFMA and the rest. Each MFMA
      // then has vector work behind it.
      const int ks = sl / NDB, part = sl % NDB;  // P step and share exponentiated here
      float xv[VPS];
      auto expo = [&](int w) {  // exponentials of word w of this slot's share
        const int t = part * VPS + 2 * w;
        xv[2 * w] = __builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][(ks & 1) * 8 + t], c2, -ms));
        xv[2 * w + 1] = __builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][(ks & 1) * 8 + t + 1], c2, -ms));
      };
      // bf16 pair for P.V, and the row sum of the fp32 values. The sum is two
      // plain adds: v_dot2_f32_bf16 on the packed pair, one instruction instead
      // of two, stalls the matrix unit when issued between MFMAs (measured on
      // this chip: one per MFMA slows a stream of MFMAs by 50-70%)
      auto pack = [&](int w) {
        const int t = part * VPS + 2 * w;
        typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
        const bf16x2v pr = {(__bf16)xv[2 * w], (__bf16)xv[2 * w + 1]};
        const uint32_t word = __builtin_bit_cast(uint32_t, pr);
        pw[ks][t / 2] = word;
        rs0 += xv[2 * w];
        rs1 += xv[2 * w + 1];
      };
      constexpr int WPS = VPS / 2, WA = (WPS + 1) / 2;  // words per slot, words in the first half
      if (sl < NM) {
        const int g = sl / (QF_ * GB), kk = (sl % (QF_ * GB)) / GB, kb = g * GB + sl % GB;
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[sl], qf.f[kk], kk == 0 ? f32x16{} : sn[kb], 0, 0, 0);
#pragma unroll
        for (int w = 0; w < WA; ++w) expo(w);
        if (WPS > 1) {
#pragma unroll
          for (int w = 0; w < WA; ++w) pack(w);
          asm volatile("" : "+v"(rs0), "+v"(rs1));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (sl >= NDB) {
        const int pi = sl - NDB, pks = pi / NDB, db = pi % NDB;
        const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[pks][0], pw[pks][1], pw[pks][2], pw[pks][3]});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[sl], pf, o[db], 0, 0, 0);
      }
      if (sl < NM) {
        if (WPS == 1) {
          pack(0);
        } else {
#pragma unroll
          for (int w = WA; w < WPS; ++w) {
            expo(w);
            pack(w);
          }
        }
      }
      // lane maxima: group g finished at slot fin = (g + 1) * QF * GB - 1; its
      // 16 * GB values per lane are spread over the slots after fin + 1 (the
      // last group over the remaining slots from fin + 1)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int fin = (g + 1) * QF_ * GB - 1;
        const int first = (g == NG - 1) ? fin + 1 : fin + 2;
        const int last = (g == NG - 1) ? NSL - 1 : (g + 2) * QF_ * GB - 1;
        if (sl >= first && sl <= last) {
          constexpr int NV = 16 * GB;
          const int nsl = last - first + 1, k = sl - first;
          const int v0 = NV * k / nsl, v1 = NV * (k + 1) / nsl;
#pragma unroll
          for (int v = v0; v < v1; ++v) {
            const float x = sn[g * GB + v / 16][v % 16];
            mx[g][v & 1] = fmax_raw(mx[g][v & 1], x);
          }
          asm volatile("" : "+v"(mx[g][0]), "+v"(mx[g][1]));
        }
      }
      // the row sums and maxima have no use inside the phase: without these
      // empty uses they would all be computed after its last MFMA
      if (sl < NM) asm volatile("" : "+v"(rs0), "+v"(rs1));
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = fmaf(l_run, alpha, rs0 + rs1);
    float mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g) mt = fmax_raw(mt, fmax_raw(mx[g][0], mx[g][1]));
    mt_out = mt;
  };

  // Keys of tile t (first key at position pos0, then every kps positions) that
  // this lane may see: those with index <= the returned bound (minus 4h, the
  // lane's offset inside each group of 8 keys). Key i is visible when
  // pos0 + kps * i <= qpos, i.e. i <= floor((qpos - pos0) / kps).
  auto key_bound = [&](int t, int pos0) {
    const int nvalid = (int)min((int64_t)TB, p.Lk - (int64_t)t * TB);
    int rel = wk.qpos < pos0 ? -1 : wk.qpos - pos0;
    // floor(rel / kps) for 0 <= rel < 2^31 as (rel + 1/2) / kps in fp64: the
    // exact quotient lies at least 1/(2 kps) from an integer, and the product's
    // error is below 2^31 / kps * 2^-51, so truncation gives the floor exactly
    if constexpr (MASK == 2) rel = rel < 0 ? -1 : (int)__builtin_fma((double)rel, p.kinv, 0.5 * p.kinv);
    return min(rel, nvalid - 1) - 4 * h;
  };
  // Keys outside [lo, bound] (both minus 4h) are masked; lo only on block-sparse calls.
  // The test is lane-local integer arithmetic: the sign of bound - key is spread
  // over the word and selects the bits of -inf. Written as compares, every
  // element's result took a scalar register pair, and the spills of the walk
  // state this forced ran on every step, masked or not. The empty asm keeps the
  // compiler from turning the selects back into compares whose results it holds
  // in scalar registers.
  auto mask_tile = [&](f32x16* s, int bound, int lo) {
#pragma unroll
    for (int k2 = 0; k2 < TB / 32; ++k2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k2 * 32 + 8 * (r >> 2) + (r & 3);
        int hide = (bound - key) >> 31;  // all ones when key > bound
        if constexpr (SP) hide |= (key - lo) >> 31;
        asm volatile("" : "+v"(hide));
        const float sv = s[k2][r];  // copy first: a bit cast of the element itself reads element 0
        const uint32_t bits = __builtin_bit_cast(uint32_t, sv);
        s[k2][r] = __builtin_bit_cast(float, (bits & ~(uint32_t)hide) | ((uint32_t)hide & 0xff800000u));
      }
  };
  // Block-sparse calls: the run of keys of the tile starting at position pos0
  // that the block mask admits for this wave, packed as (lo << 16) | (hi + 1)
  // (empty: lo = TB, hi = -1). The tile's keys are pos0 .. pos0 + TB - 1 and
  // key blocks are at least TB long, so the tile meets blocks kb0 and kb0 + 1.
  auto sparse_run = [&](int pos0) {
    if constexpr (!SP) {
      return (int)TB;
    } else {
      const int kb0 = pos0 >> p.sp_lgk;
      const uint32_t* row = p.sp_bits + (int64_t)wqb * p.sp_rw + (kb0 >> 5);
      const uint32_t w0 = cload(row), w1 = cload(row + 1);
      const int sh = kb0 & 31;
      const bool b0 = (w0 >> sh) & 1u;
      const bool b1 = sh == 31 ? (w1 & 1u) : ((w0 >> (sh + 1)) & 1u);
      const int split = ((kb0 + 1) << p.sp_lgk) - pos0;  // first key of block kb0 + 1
      int lo = TB, hi = -1;
      if (split >= TB) {
        if (b0) lo = 0, hi = TB - 1;
      } else if (b0 && b1) {
        lo = 0, hi = TB - 1;
      } else if (b0) {
        lo = 0, hi = split - 1;
      } else if (b1) {
        lo = split, hi = TB - 1;
      }
      return (lo << 16) | (hi + 1);
    }
  };

  uint32_t off[O::NS];
  int off_ss = -1;
  auto stage = [&](const TileInfo& t, bool is_v, char* dst) {
    if (fast_tile(p, t, DP)) {
      if (t.ss != off_ss) {
        off_ss = t.ss;
#pragma unroll
        for (int i = 0; i < O::NS; ++i) off[i] = O::piece_offset(i, tid, 2u * (uint32_t)t.ss);
      }
      O::copy_fast(is_v ? t.vp : t.kp, off, dst, wave);
    } else {
      O::template copy_slow<MODE>(p, t, b, hk, tid, wave, is_v, dst);
    }
  };

  // Copies into LDS go out in groups: group i = {K(i+1+D), V(i+D)}, issued at
  // iteration i (the prologue issues K(0) and the groups i = -D .. -1).
  // Iteration j needs group j-D; the D-1 groups issued after it may still be
  // in flight when they are whole, i.e. when tile j+D exists.
  constexpr int kGroupOps = 2 * O::NS;
  auto wait_group = [&](bool later_groups_whole) {
    if (later_groups_whole)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * kGroupOps));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  // the work item's tiles: the dense walk, or entries of its list on block-sparse calls
  SparseWalk sw = {nullptr, 0};
  int e0 = 0;
  if constexpr (SP) {
    sw.list = p.sp_list + (int64_t)wk.qt * p.sp_cap;
    const int cnt = cload(p.sp_count + wk.qt);
    e0 = lower_entry(sw.list, cnt, tbeg);
    sw.end = lower_entry(sw.list, cnt, tend);
  }
  auto next_of = [&](const TileInfo& x) {
    if constexpr (SP)
      return uniform(sparse_successor<MODE, 2, TB, false>(p, sw, x, tend, wk.gqmax, b, hk));
    else
      return uniform(successor<MODE, 2, TB, false>(p, x, tend, wk.gqmax, b, hk));
  };
  const TileInfo t0 = SP ? uniform(sparse_tile<MODE, 2, TB, false>(p, sw, e0, 0, tend, wk.gqmax, b, hk))
                         : uniform(next_tile<MODE, 2, TB, true, false>(p, tbeg, 0, tend, wk.gqmax, b, hk));
  if (t0.t < tend) {
    f32x16 sa[TB / 32], sb[TB / 32];
    // Tile index and first position of tiles j .. j+D, in slot (tile mod NB),
    // and (block-sparse calls) the run of keys the block mask admits.
    int qt[NB], qp[NB], qm[NB];

    // Prologue: K(0), then groups {K(k+1), V(k)} for k < D.
    qt[0] = t0.t;
    qp[0] = t0.pos0;
    qm[0] = sparse_run(t0.pos0);
    stage(t0, false, kbuf[0]);
    TileInfo tv = t0;
    TileInfo tk = next_of(t0);
#pragma unroll
    for (int k = 0; k < D; ++k) {
      qt[k + 1] = tk.t;
      qp[k + 1] = tk.pos0;
      qm[k + 1] = sparse_run(tk.pos0);
      if (tk.t < tend) stage(tk, false, kbuf[k + 1]);
      if (tv.t < tend) stage(tv, true, vbuf[k]);
      tv = tk;
      if (tk.t < tend) tk = next_of(tk);
    }
    // K(0) has landed once at most the D groups after it are in flight.
    if (qt[D] < tend)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(D * kGroupOps));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    O::qk(kbuf[0], qf, L, sa);
    if constexpr (MASK) {
      int hi = key_bound(qt[0], qp[0]), lo = 0;
      if constexpr (SP) {
        hi = min(hi, (qm[0] & 0xffff) - 1 - 4 * h);
        lo = (qm[0] >> 16) - 4 * h;
      }
      mask_tile(sa, hi, lo);
    }
    float mt = lane_max(sa);  // lane maximum of the scores of the next tile to exponentiate

    // Iteration j (BI = j mod NB): scores of tile j in sc, of tile j+1 into sn.
    // After the last tile the scores of a missing tile j+1 are computed from
    // stale LDS and never used: the loop body stays the same for every tile.
    // The four ring buffers of a step are passed as restrict pointers: the
    // compiler then knows that the reads of K(j+1) and V(j) do not touch the
    // buffers being filled, and does not make them wait for those copies.
    auto step_body = [&](f32x16* sc, f32x16* sn, auto bi_c, auto mask_c, bool need, int tn, int pn, int mrun,
                         char* __restrict__ k_fill, char* __restrict__ v_fill, const char* __restrict__ k_read,
                         const char* __restrict__ v_read) {
      constexpr int BI = decltype(bi_c)::value;
      constexpr bool MASKED = decltype(mask_c)::value != 0;
      wait_group(qt[(BI + D) % NB] < tend);  // K(j+1) and V(j) have landed
      __syncthreads();
      finish_max(mt, true);  // reference for tile j
      rescale_o();           // o to that reference
      qt[BI] = tk.t;
      qp[BI] = tk.pos0;
      if constexpr (SP) qm[BI] = sparse_run(tk.pos0);
      if (tk.t < tend) stage(tk, false, k_fill);  // K(j+1+D)
      if (tv.t < tend) stage(tv, true, v_fill);   // V(j+D)
      __builtin_amdgcn_sched_barrier(0);
      // the phase of matrix and softmax work runs at raised wave priority, so the SIMD's arbiter
      // prefers it to the other wave's copy issue and barrier wait (+0.5-1% measured)
      __builtin_amdgcn_s_setprio(1);
      fused(k_read, v_read, sc, sn, mt);
      __builtin_amdgcn_s_setprio(0);
      // some lane of the wave may not see every key of tile j+1: mask, and take
      // the maximum again (the masked maximum never exceeds the one above)
      if (MASKED && need) {
        int bound = key_bound(tn, pn), lo = 0;
        if constexpr (SP) {
          bound = min(bound, (mrun & 0xffff) - 1 - 4 * h);
          lo = (mrun >> 16) - 4 * h;
        }
        mask_tile(sn, bound, lo);
        mt = fminf(mt, lane_max(sn));
      }
      tv = tk;
      if (tk.t < tend) tk = next_of(tk);
    };
    auto step = [&](f32x16* sc, f32x16* sn, auto bi_c) {
      constexpr int BI = decltype(bi_c)::value;
      const int tn = qt[(BI + 1) % NB], pn = qp[(BI + 1) % NB];
      // A uniform test (scalar work) of whether some lane of the wave may not see every key of tile
      // j+1: a ragged last tile, or the wave's earliest query before the tile's last key (key i sits
      // at pos0 + kps i). It may say yes where every lane sees every key, never the reverse; the
      // per-lane bound is formed only then.
      bool need = false;
      int mrun = 0;
      if constexpr (MASK) {
        const int64_t nvalid = min((int64_t)TB, p.Lk - (int64_t)tn * TB);
        need = nvalid < TB || (int64_t)wk.wqmin - pn < (int64_t)p.kps * (TB - 1);
      }
      if constexpr (SP) {
        // the block mask's run of admitted keys: anything short of the whole tile needs the mask
        mrun = qm[(BI + 1) % NB];
        need = need || (mrun >> 16) > 0 || (mrun & 0xffff) < TB;
      }
      step_body(sc, sn, bi_c, IntC<MASK>{}, need, tn, pn, mrun, kbuf[BI], vbuf[(BI + D) % NB],
                kbuf[(BI + 1) % NB], vbuf[BI]);
    };

    while (true) {
      step(sa, sb, IntC<0>{});
      if (qt[1 % NB] >= tend) break;
      step(sb, sa, IntC<1>{});
      if (qt[2 % NB] >= tend) break;
      if constexpr (NB == 4) {
        step(sa, sb, IntC<2>{});
        if (qt[3] >= tend) break;
        step(sb, sa, IntC<3>{});
        if (qt[0] >= tend) break;
      }
    }
  }

  write_rows<DP, MODE>(p, wk, o, l_run, m_ref, m_max, h);
}

// Merge of the key-range partials of each row, in range order, then u / l and
// lse (ring call), or, with STATS, the merged statistics themselves: u and l
// relative to the row's overall maximum, written to out and lse, and that
// maximum in score units to mout (chunk-statistics call).
// Each row is handled by LPR lanes of one wave; with VEC4 (head_dim a multiple
// of 4) each lane reads and writes 16-byte column groups.
template <bool VEC4, bool STATS>
__global__ __launch_bounds__(256) void combine_kernel(int64_t rows, int d, int nsplit, int lpr, int lpr_shift,
                                                      const float* __restrict__ part, float* __restrict__ out,
                                                      float* __restrict__ lse, float* __restrict__ mout, float c2,
                                                      float scale) {
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> lpr_shift;
  if (r >= rows) return;
  const int sub = threadIdx.x & (lpr - 1);
  const float* pl = part + (int64_t)nsplit * rows * d;
  const float* pm = pl + (int64_t)nsplit * rows;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, pm[(int64_t)s * rows + r]);
  const float ms = (mx == -INFINITY) ? 0.f : mx * c2;
  float l = 0.f;
  if (VEC4) {
    const int n4 = d >> 2;
    for (int c = sub; c < n4; c += lpr) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      float lc = 0.f;
#pragma unroll 4
      for (int s = 0; s < nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f(pm[(int64_t)s * rows + r] * c2 - ms);
        lc = fmaf(pl[(int64_t)s * rows + r], w, lc);
        u += ((const f32x4*)(part + ((int64_t)s * rows + r) * d))[c] * w;
      }
      l = lc;  // lane 0 of the row always has column group 0
      const float inv = STATS ? 1.f : ((lc > 0.f) ? 1.f / lc : 0.f);
      ((f32x4*)(out + r * d))[c] = u * inv;
    }
  } else {
    for (int s = 0; s < nsplit; ++s)
      l = fmaf(pl[(int64_t)s * rows + r], __builtin_amdgcn_exp2f(pm[(int64_t)s * rows + r] * c2 - ms), l);
    const float inv = STATS ? 1.f : ((l > 0.f) ? 1.f / l : 0.f);
    for (int c = sub; c < d; c += lpr) {
      float u = 0.f;
      for (int s = 0; s < nsplit; ++s)
        u = fmaf(part[((int64_t)s * rows + r) * d + c], __builtin_amdgcn_exp2f(pm[(int64_t)s * rows + r] * c2 - ms),
                 u);
      out[r * d + c] = u * inv;
    }
  }
  if (sub == 0) {
    if (STATS) {
      lse[r] = l;
      mout[r] = (mx == -INFINITY) ? -INFINITY : mx * scale;
    } else if (lse != nullptr) {
      lse[r] = (l > 0.f) ? mx * scale + logf(l) : -INFINITY;
    }
  }
}

// Launch of combine_kernel over `rows` rows of head_dim d.
template <bool STATS>
hipError_t launch_combine(int64_t rows, int d, int nsplit, const float* part, float* out, float* lse, float* mout,
                          float c2, float scale, hipStream_t s) {
  const bool vec4 = d % 4 == 0 && (uintptr_t)out % 16 == 0;  // partials are 256-byte aligned
  const int cols = vec4 ? d / 4 : d;
  int lpr = 1, sh = 0;
  while (lpr < cols && lpr < 64) {
    lpr <<= 1;
    ++sh;
  }
  const int64_t cblocks = (rows * lpr + 255) / 256;
  if (vec4)
    hipLaunchKernelGGL((combine_kernel<true, STATS>), dim3((unsigned)cblocks), dim3(256), 0, s, rows, d, nsplit, lpr,
                       sh, part, out, lse, mout, c2, scale);
  else
    hipLaunchKernelGGL((combine_kernel<false, STATS>), dim3((unsigned)cblocks), dim3(256), 0, s, rows, d, nsplit,
                       lpr, sh, part, out, lse, mout, c2, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of two statistics, in place on the accumulator. Each row is handled by
// LPR lanes of one wave (LPR divides 64), so every lane of a row has loaded the
// old m and l before the row's first lane overwrites them.

template <bool VEC4>
__global__ __launch_bounds__(256) void merge_kernel(int64_t rows, int d, int lpr, int lpr_shift,
                                                    float* __restrict__ au, float* __restrict__ al,
                                                    float* __restrict__ am, const float* __restrict__ bu,
                                                    const float* __restrict__ bl,
                                                    const float* __restrict__ bm) {
  const int64_t gthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t rows_per_pass = gthreads >> lpr_shift;
  const int sub = threadIdx.x & (lpr - 1);
  for (int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> lpr_shift; r < rows;
       r += rows_per_pass) {
    const float ma = am[r], mb = bm[r];
    const float la = al[r], lb = bl[r];
    const float mx = fmaxf(ma, mb);
    float fa = 0.f, fb = 0.f;
    if (mx != -INFINITY) {
      fa = expf(ma - mx);
      fb = expf(mb - mx);
    }
    // every byte of u is touched once: non-temporal loads and stores keep the
    // stream out of the caches (+16% on 1.6 GB of rotating statistics, where the
    // plain accesses ran at a device copy's rate)
    if (VEC4) {
      const int n4 = d >> 2;
      f32x4* pa = (f32x4*)(au + r * d);
      const f32x4* pb = (const f32x4*)(bu + r * d);
      for (int c = sub; c < n4; c += lpr) {
        const f32x4 x = __builtin_nontemporal_load(pa + c), y = __builtin_nontemporal_load(pb + c);
        __builtin_nontemporal_store(x * fa + y * fb, pa + c);
      }
    } else {
      float* pa = au + r * d;
      const float* pb = bu + r * d;
      for (int c = sub; c < d; c += lpr)
        __builtin_nontemporal_store(__builtin_nontemporal_load(pa + c) * fa + __builtin_nontemporal_load(pb + c) * fb,
                                    pa + c);
    }
    if (sub == 0) {
      am[r] = mx;
      al[r] = la * fa + lb * fb;
    }
  }
}

// ---------------------------------------------------------------------------
// Block-sparse planning. The caller's mask is a byte matrix over (query block,
// key block) of global positions. sparse_bits_kernel packs it 32 key blocks per
// word (row stride rw words, the last word of a row zero, so a two-word read
// at any key block of the row stays inside it). sparse_plan_kernel then lists,
// for each query tile of bm rows, the key tiles of tb keys that hold at least
// one pair the mask (and, when causal, the positions) allow, in ascending
// order. Position runs with a step other than 1 are treated as their whole
// interval, which can only add tiles, never drop one.

__global__ __launch_bounds__(256) void sparse_bits_kernel(const uint8_t* __restrict__ mask, int64_t nqb, int64_t nkb,
                                                          int rw, uint32_t* __restrict__ words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nqb * rw) return;
  const int64_t a = i / rw;
  const int64_t kb0 = (i % rw) * 32;
  uint32_t bits = 0;
  for (int j = 0; j < 32; ++j)
    if (kb0 + j < nkb && mask[a * nkb + kb0 + j] != 0) bits |= 1u << j;
  words[i] = bits;
}

constexpr int kPlanParts = 8;  // query position runs kept per query tile (more are merged into the last)

// Is some pair of a query in [qlo, qhi] and a key in [klo, khi] allowed?
__device__ __forceinline__ bool runs_meet(const uint32_t* __restrict__ words, int rw, int lgq, int lgk, bool causal,
                                          int qlo, int qhi, int klo, int khi) {
  if (causal && klo > qhi) return false;
  const int qa = qlo >> lgq, qz = qhi >> lgq, ka = klo >> lgk, kz = khi >> lgk;
  if ((int64_t)(qz - qa + 1) * (kz - ka + 1) > 4096) return true;  // too many blocks to check: keep the tile
  for (int qb = qa; qb <= qz; ++qb) {
    const uint32_t* row = words + (int64_t)qb * rw;
    const int64_t qmax = min((int64_t)qhi, (((int64_t)qb + 1) << lgq) - 1);
    for (int kb = ka; kb <= kz; ++kb) {
      if (!((row[kb >> 5] >> (kb & 31)) & 1u)) continue;
      if (!causal || max((int64_t)klo, (int64_t)kb << lgk) <= qmax) return true;
    }
  }
  return false;
}

__global__ __launch_bounds__(256) void sparse_plan_kernel(const ChunkDev* __restrict__ chunks, int n_chunks,
                                                          const QSegDev* __restrict__ qsegs, int n_qseg, int64_t lq,
                                                          int64_t lk, int bm, int tb, const uint32_t* __restrict__ words,
                                                          int rw, int lgq, int lgk, int causal, int cap,
                                                          int* __restrict__ list, int* __restrict__ count) {
  __shared__ int qlo_s[kPlanParts], qhi_s[kPlanParts];
  __shared__ int nparts_s;
  __shared__ int wsum[4];
  const int qt = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    // position runs of this query tile's rows, one per query segment it meets
    int np = 0;
    const int64_t r0 = (int64_t)qt * bm, r1 = min(lq, r0 + bm);
    for (int s = 0; s < n_qseg; ++s) {
      const QSegDev g = qsegs[s];
      const int64_t a = max(r0, g.row0), e = min(r1, g.row0 + g.len);
      if (a >= e) continue;
      const int lo = (int)(g.pos0 + g.ps * (a - g.row0)), hi = (int)(g.pos0 + g.ps * (e - 1 - g.row0));
      if (np < kPlanParts) {
        qlo_s[np] = lo;
        qhi_s[np] = hi;
        ++np;
      } else {
        qlo_s[np - 1] = min(qlo_s[np - 1], lo);
        qhi_s[np - 1] = max(qhi_s[np - 1], hi);
      }
    }
    nparts_s = np;
  }
  __syncthreads();
  const int np = nparts_s;
  const int ntiles = (int)((lk + tb - 1) / tb);
  const int wave = tid >> 6, lane = tid & 63;
  int running = 0;
  for (int base = 0; base < ntiles; base += 256) {
    const int t = base + tid;
    bool vis = false;
    if (t < ntiles) {
      int64_t j0 = (int64_t)t * tb;
      const int64_t j1 = min(lk, j0 + tb);
      int lo = 0, hi = n_chunks - 1;  // last chunk starting at or before key j0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunks[mid].start <= j0) lo = mid; else hi = mid - 1;
      }
      for (int c = lo; j0 < j1 && c < n_chunks && !vis; ++c) {
        const ChunkDev ch = chunks[c];
        const int64_t e = min(j1, ch.start + ch.len);
        if (e <= j0) continue;
        const int klo = ch.pos0 + ch.ps * (int)(j0 - ch.start), khi = ch.pos0 + ch.ps * (int)(e - 1 - ch.start);
        for (int i = 0; i < np && !vis; ++i)
          vis = runs_meet(words, rw, lgq, lgk, causal != 0, qlo_s[i], qhi_s[i], klo, khi);
        j0 = e;
      }
    }
    // compact in tile order: ballot within each wave, wave totals through LDS
    const uint64_t bal = __ballot(vis);
    const int before = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (vis) list[(int64_t)qt * cap + off + before] = t;
    running += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) count[qt] = running;
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side: validation, descriptor tables, dispatch. The helpers in ra_host
// are shared with the backward pass (host_common.h).

namespace ra_host {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) { return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e)); }

int check_dims(int dtype, int batch, int q_heads, int kv_heads, int head_dim) {
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0)
    return fail(RA_ERR_SHAPE, "batch=%d q_heads=%d kv_heads=%d", batch, q_heads, kv_heads);
  if (q_heads % kv_heads != 0)
    return fail(RA_ERR_SHAPE, "q_heads=%d is not a multiple of kv_heads=%d", q_heads, kv_heads);
  if (head_dim < 1 || head_dim > 128) return fail(RA_ERR_UNSUPPORTED, "head_dim=%d outside 1..128", head_dim);
  return RA_OK;
}

// Position step of a chunk or query segment: 0 stands for 1 (contiguous).
int64_t pos_step(int64_t s) { return s == 0 ? 1 : s; }

// True when offset, offset + step, ..., offset + step * (len - 1) all lie in
// [0, kPosLimit] (len >= 1, step >= 1).
bool positions_fit(int64_t offset, int64_t len, int64_t step) {
  if (offset < 0 || offset > kPosLimit || step < 1 || step > kPosLimit) return false;
  return len - 1 <= (kPosLimit - offset) / step;
}

int check_chunk(const ra_kv_chunk& c, int idx, int head_dim) {
  if (c.len < 0) return fail(RA_ERR_SHAPE, "chunk %d: negative length", idx);
  if (c.pos_stride < 0) return fail(RA_ERR_SHAPE, "chunk %d: negative pos_stride", idx);
  if (c.len == 0) return RA_OK;
  if (!c.k || !c.v) return fail(RA_ERR_NULL, "chunk %d: null k or v", idx);
  if (!positions_fit(c.global_offset, c.len, pos_step(c.pos_stride)))
    return fail(RA_ERR_SHAPE, "chunk %d: positions %lld + %lld * [0, %lld) outside [0, 2^31-1)", idx,
                (long long)c.global_offset, (long long)pos_step(c.pos_stride), (long long)c.len);
  if (c.stride_s < head_dim || c.stride_b < 0 || c.stride_h < 0)
    return fail(RA_ERR_SHAPE, "chunk %d: strides b=%lld h=%lld s=%lld invalid for head_dim %d", idx,
                (long long)c.stride_b, (long long)c.stride_h, (long long)c.stride_s, head_dim);
  return RA_OK;
}

bool vec_ok(const void* p, int64_t stride, int head_dim, int64_t elem) {
  const int64_t per16 = 16 / elem;
  return ((uintptr_t)p % 16 == 0) && stride % per16 == 0 && head_dim % per16 == 0;
}

bool chunk_vec_ok(const ra_kv_chunk& c, int head_dim, int64_t elem) {
  if (c.len == 0) return true;
  const int64_t per16 = 16 / elem;
  return vec_ok(c.k, c.stride_s, head_dim, elem) && vec_ok(c.v, c.stride_s, head_dim, elem) &&
         c.stride_b % per16 == 0 && c.stride_h % per16 == 0;
}

}  // namespace ra_host

namespace {
using namespace ra_host;

int dp_of(int head_dim) { return head_dim <= 32 ? 32 : (head_dim <= 64 ? 64 : 128); }

// The forward kernels' tile walk keeps a chunk's row stride (in elements) in
// 32 bits.
int check_row_stride(const ra_kv_chunk& c, int idx) {
  if (c.len > 0 && c.stride_s > 0x7fffffffLL)
    return fail(RA_ERR_UNSUPPORTED, "chunk %d: row stride %lld elements is 2^31 or more", idx,
                (long long)c.stride_s);
  return RA_OK;
}

// Key-range split for grids that cannot fill the chip: depends only on the
// shape (never on the chunk list), so every split of a sequence into chunks
// runs the same arithmetic.
// `resident`: workgroups of the kernel that fit on one CU at a time; `rounds`:
// how many times over the grid should fill the chip (2 balances the unequal
// work of causal query tiles; equal work needs 1).
int choose_nsplit(int64_t base_blocks, int64_t lk, int resident, int rounds) {
  const int64_t ntiles = (lk + BN - 1) / BN;
  const int64_t target = 256 * resident * rounds;
  if (base_blocks >= 256 * resident) return 1;  // one full round already
  int64_t s = (target + base_blocks - 1) / base_blocks;
  const int64_t max_by_work = ntiles / 16;  // keep at least 16 tiles per range
  if (s > max_by_work) s = max_by_work;
  if (s > 32) s = 32;
  return s < 1 ? 1 : (int)s;
}

template <class T, int DP, int MODE>
hipError_t launch_t(const Params& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((attention_kernel<T, DP, MODE>), dim3(nblocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int DP, int MODE>
hipError_t launch_pipe(const Params& p, bool mask, int nblocks, hipStream_t s) {
  constexpr int nt = 64 * pipe_waves(MODE);
  if (mask && MODE == kRingCausal && p.kps != 1) {
    if constexpr (MODE == kRingCausal)
      hipLaunchKernelGGL((attention_bf16_kernel<DP, MODE, 2>), dim3(nblocks), dim3(nt), 0, s, p);
  } else if (mask) {
    hipLaunchKernelGGL((attention_bf16_kernel<DP, MODE, 1>), dim3(nblocks), dim3(nt), 0, s, p);
  } else {
    hipLaunchKernelGGL((attention_bf16_kernel<DP, MODE, 0>), dim3(nblocks), dim3(nt), 0, s, p);
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int dtype, int dp, const Params& p, int nblocks, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (dp == 32) return launch_t<__bf16, 32, MODE>(p, nblocks, s);
    if (dp == 64) return launch_t<__bf16, 64, MODE>(p, nblocks, s);
    return launch_t<__bf16, 128, MODE>(p, nblocks, s);
  }
  if (dp == 32) return launch_t<float, 32, MODE>(p, nblocks, s);
  if (dp == 64) return launch_t<float, 64, MODE>(p, nblocks, s);
  return launch_t<float, 128, MODE>(p, nblocks, s);
}

template <int MODE>
hipError_t launch_pipe_mode(int dp, const Params& p, bool mask, int nblocks, hipStream_t s) {
  if (dp == 32) return launch_pipe<32, MODE>(p, mask, nblocks, s);
  if (dp == 64) return launch_pipe<64, MODE>(p, mask, nblocks, s);
  return launch_pipe<128, MODE>(p, mask, nblocks, s);
}

// pipe: the pipelined bf16 kernel applies (see pipe_ok); mask: it needs the
// position mask on every tile.
hipError_t launch(int mode, int dtype, int dp, const Params& p, bool pipe, bool mask, int nblocks, hipStream_t s) {
  if (pipe) {
    if (mode == kStats) return launch_pipe_mode<kStats>(dp, p, mask, nblocks, s);
    if (mode == kRingFull) return launch_pipe_mode<kRingFull>(dp, p, mask, nblocks, s);
    return launch_pipe_mode<kRingCausal>(dp, p, mask, nblocks, s);
  }
  if (mode == kStats) return launch_mode<kStats>(dtype, dp, p, nblocks, s);
  if (mode == kRingFull) return launch_mode<kRingFull>(dtype, dp, p, nblocks, s);
  return launch_mode<kRingCausal>(dtype, dp, p, nblocks, s);
}

// Block-sparse variants: the pipelined kernel (MASK = 1 with the block run) or
// the general kernel with the per-score block check.
template <int DP, int MODE>
hipError_t launch_sparse_dp(int dtype, bool pipe, const Params& p, int nblocks, hipStream_t s) {
  if (pipe)
    hipLaunchKernelGGL((attention_bf16_kernel<DP, MODE, 1, true>), dim3(nblocks), dim3(64 * pipe_waves(MODE)), 0, s,
                       p);
  else if (dtype == RA_BF16)
    hipLaunchKernelGGL((attention_kernel<__bf16, DP, MODE, true>), dim3(nblocks), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((attention_kernel<float, DP, MODE, true>), dim3(nblocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_sparse_mode(int dtype, int dp, bool pipe, const Params& p, int nblocks, hipStream_t s) {
  if (dp == 32) return launch_sparse_dp<32, MODE>(dtype, pipe, p, nblocks, s);
  if (dp == 64) return launch_sparse_dp<64, MODE>(dtype, pipe, p, nblocks, s);
  return launch_sparse_dp<128, MODE>(dtype, pipe, p, nblocks, s);
}


// The pipelined bf16 kernel copies whole 16-byte pieces into LDS with 32-bit
// lane offsets and masks by key index within a tile, so it needs: bf16,
// head_dim a multiple of 8, 16-byte aligned rows, row offsets inside a tile
// below 2^31 bytes, and (when causal) one position step shared by every chunk
// (returned in *kps) with positions that continue the progression across
// every chunk boundary that falls inside a tile.
bool pipe_ok(int dtype, int head_dim, bool vec, const ra_kv_chunk* chunks, int n_chunks, bool causal, int* kps) {
  *kps = 1;
  if (dtype != RA_BF16 || head_dim % 8 != 0 || !vec) return false;
  const int tb = pipe_tile(dp_of(head_dim));
  int64_t start = 0, step = 0;
  const ra_kv_chunk* prev = nullptr;
  for (int c = 0; c < n_chunks; ++c) {
    const ra_kv_chunk& ch = chunks[c];
    if (ch.len == 0) continue;
    if ((int64_t)tb * ch.stride_s * 2 >= ((int64_t)1 << 31)) return false;
    if (causal) {
      const int64_t s = pos_step(ch.pos_stride);
      if (step != 0 && s != step) return false;
      step = s;
      if (prev && start % tb != 0 && ch.global_offset != prev->global_offset + step * prev->len) return false;
    }
    start += ch.len;
    prev = &ch;
  }
  if (step != 0) *kps = (int)step;
  return true;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t table_bytes(int n_chunks, int n_q_segments) {
  return align256(sizeof(ChunkDev) * (size_t)n_chunks) + align256(sizeof(QSegDev) * (size_t)n_q_segments);
}

size_t partial_bytes(int nsplit, int64_t rows, int head_dim) {
  return nsplit > 1 ? align256(sizeof(float) * (size_t)nsplit * (size_t)rows * (size_t)(head_dim + 2)) : 0;
}

}  // namespace

extern "C" {

const char* ra_status_string(int status) {
  switch (status) {
    case RA_OK: return "ok";
    case RA_ERR_NULL: return "null pointer";
    case RA_ERR_SHAPE: return "invalid shape";
    case RA_ERR_DTYPE: return "invalid dtype";
    case RA_ERR_UNSUPPORTED: return "unsupported";
    case RA_ERR_HIP: return "HIP runtime error";
    case RA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* ra_last_error(void) { return g_err; }

size_t ra_ring_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                               int n_chunks, int n_q_segments) {
  if (n_chunks < 0) n_chunks = 0;
  if (n_q_segments < 0) n_q_segments = 0;
  size_t bytes = table_bytes(n_chunks, n_q_segments) + 256;
  if (batch > 0 && q_heads > 0 && q_len > 0 && head_dim > 0 && total_keys > 0) {
    // room for the larger of the two kernels' key-range splits
    const int64_t base = ((q_len + BM - 1) / BM) * (int64_t)q_heads * batch;
    const int bmp = pipe_bm(kRingFull);
    const int64_t base_pipe = ((q_len + bmp - 1) / bmp) * (int64_t)q_heads * batch;
    const int ns =
        max(choose_nsplit(base, total_keys, 2, 2), choose_nsplit(base_pipe, total_keys, pipe_resident(kRingFull), 2));
    bytes += partial_bytes(ns, (int64_t)batch * q_heads * q_len, head_dim);
  }
  return bytes;
}

// ---------------------------------------------------------------------------
}  // extern "C"

// Measurement hook: HIP events recorded on the call's stream right before and
// after the attention kernel of each ring_attention / attention_chunk_stats
// call (not around the key-range combine), and around the two gradient
// kernels of each ring_attention_backward call, while enabled.
namespace ra_host {

// Descriptor tables travel to the device as kernel arguments: 2 KB per launch,
// well inside the kernel argument space.
__global__ __launch_bounds__(256) void upload_kernel(uint32_t* __restrict__ dst, int n, UploadWindow a) {
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = a.w[i];
}

void TableUpload::flush() {
  if (fill_ == 0) return;
  hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, s_, (uint32_t*)(dst_ + base_), (int)(fill_ / 4), win_);
  const hipError_t e = hipGetLastError();
  if (err_ == hipSuccess) err_ = e;
  base_ += fill_;
  fill_ = 0;
}

void TableUpload::put(const void* p, size_t n) {
  const char* src = (const char*)p;
  while (n > 0) {
    const size_t room = sizeof(win_) - fill_;
    const size_t k = n < room ? n : room;
    memcpy((char*)win_.w + fill_, src, k);
    fill_ += k;
    src += k;
    n -= k;
    if (fill_ == sizeof(win_)) flush();
  }
}

void TableUpload::zero_to(size_t total) {
  static const uint32_t zeros[64] = {};
  while (size() < total) {
    const size_t k = total - size() < sizeof(zeros) ? total - size() : sizeof(zeros);
    put(zeros, k);
  }
}

hipError_t TableUpload::finish() {
  flush();
  return err_;
}

constexpr int kTimerSlots = 512;
hipEvent_t g_tev[2][kTimerSlots];
bool g_tev_made = false;
int g_timer_on = 0, g_timer_n = 0;

void timer_begin(hipStream_t s) {
  if (g_timer_on && g_timer_n < kTimerSlots) (void)hipEventRecord(g_tev[0][g_timer_n], s);
}
void timer_end(hipStream_t s) {
  if (g_timer_on && g_timer_n < kTimerSlots) (void)hipEventRecord(g_tev[1][g_timer_n++], s);
}
}  // namespace ra_host

extern "C" {

int ra_kernel_timer(int enable) {
  g_err[0] = 0;
  if (enable && !g_tev_made) {
    for (int i = 0; i < kTimerSlots; ++i)
      for (int j = 0; j < 2; ++j) {
        const hipError_t e = hipEventCreate(&g_tev[j][i]);
        if (e != hipSuccess) return hip_fail(e, "kernel timer: hipEventCreate");
      }
    g_tev_made = true;
  }
  g_timer_on = enable ? 1 : 0;
  g_timer_n = 0;
  return RA_OK;
}

int ra_kernel_timer_read(float* total_ms, int* count) {
  g_err[0] = 0;
  if (!total_ms || !count) return fail(RA_ERR_NULL, "total_ms and count must be non-null");
  float tot = 0.f;
  for (int i = 0; i < g_timer_n; ++i) {
    hipError_t e = hipEventSynchronize(g_tev[1][i]);
    if (e != hipSuccess) return hip_fail(e, "kernel timer: hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_tev[0][i], g_tev[1][i]);
    if (e != hipSuccess) return hip_fail(e, "kernel timer: hipEventElapsedTime");
    tot += ms;
  }
  *total_ms = tot;
  *count = g_timer_n;
  g_timer_n = 0;
  return RA_OK;
}

size_t ra_chunk_stats_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t chunk_len) {
  if (batch <= 0 || q_heads <= 0 || head_dim <= 0 || q_len <= 0 || chunk_len <= 0) return 0;
  // both kernels take 128 query rows per workgroup in this mode. The keys are cut only while the
  // rows leave CUs idle: with one workgroup per CU already, the partial writes and the merge cost
  // more than a second workgroup per CU gains (measured on 4096 rows x 4096 keys x 8 heads)
  const int64_t base = ((q_len + BM - 1) / BM) * (int64_t)q_heads * batch;
  const int ns = choose_nsplit(base, chunk_len, 1, 1);
  return partial_bytes(ns, (int64_t)batch * q_heads * q_len, head_dim);
}

int ra_attention_chunk_stats(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                             int64_t q_len, const ra_kv_chunk* chunk, float scale, float* u, float* l, float* m,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = check_dims(dtype, batch, q_heads, kv_heads, head_dim);
  if (st) return st;
  if (!chunk) return fail(RA_ERR_NULL, "chunk descriptor is null");
  if (q_len < 0) return fail(RA_ERR_SHAPE, "q_len=%lld", (long long)q_len);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RA_ERR_SHAPE, "scale must be finite and > 0");
  const int64_t elem = dtype == RA_BF16 ? 2 : 4;
  if ((st = check_chunk(*chunk, 0, head_dim))) return st;
  if ((st = check_row_stride(*chunk, 0))) return st;
  if (q_len == 0 || batch == 0) return RA_OK;
  if (!q || !u || !l || !m) return fail(RA_ERR_NULL, "q, u, l and m must be non-null");
  if (chunk->len > kPosLimit) return fail(RA_ERR_UNSUPPORTED, "chunk longer than 2^31-2 keys");
  const bool vec = vec_ok(q, head_dim, head_dim, elem) && chunk_vec_ok(*chunk, head_dim, elem);
  int kps = 1;
  const bool pipe = pipe_ok(dtype, head_dim, vec, chunk, 1, false, &kps);
  const int bm = pipe ? pipe_bm(kStats) : BM;
  const int64_t n_qt = (q_len + bm - 1) / bm;
  const int64_t base_blocks = n_qt * q_heads * batch;
  // with a workspace, a grid too small for the chip is filled by cutting the keys into ranges whose
  // partial statistics are merged afterwards (the cut depends only on the chunk's length)
  const size_t need = ra_chunk_stats_workspace_bytes(batch, q_heads, head_dim, q_len, chunk->len);
  if (workspace && (uintptr_t)workspace % 256 != 0)
    return fail(RA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int nsplit = (need > 0 && workspace && workspace_bytes >= need)
                         ? choose_nsplit(base_blocks, chunk->len, 1, 1)
                         : 1;
  const int64_t nblocks = base_blocks * nsplit;
  if (nblocks > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid too large");

  Params p = {};
  p.q = q;
  p.o = u;
  p.l = l;
  p.m = m;
  p.part = nsplit > 1 ? (float*)workspace : nullptr;
  p.one.k = chunk->k;
  p.one.v = chunk->v;
  p.one.start = 0;
  p.one.len = chunk->len;
  p.one.sb = chunk->stride_b;
  p.one.sh = chunk->stride_h;
  p.one.ss = chunk->stride_s;
  p.one.pos0 = 0;
  p.one.ps = 1;
  p.Lq = q_len;
  p.Lk = chunk->len;
  p.n_chunks = 1;
  p.n_qseg = 0;
  p.B = batch;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.d = head_dim;
  p.n_qt = (int)n_qt;
  p.nsplit = nsplit;
  p.vec = vec;
  p.kps = kps;
  p.kinv = 1.0 / kps;
  p.scale = scale;
  p.c2 = scale * kLog2e;
  const bool mask = chunk->len % pipe_tile(dp_of(head_dim)) != 0;
  timer_begin((hipStream_t)stream);
  hipError_t e = launch(kStats, dtype, dp_of(head_dim), p, pipe, mask, (int)nblocks, (hipStream_t)stream);
  timer_end((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention_chunk_stats launch");
  if (nsplit > 1) {
    e = launch_combine<true>((int64_t)batch * q_heads * q_len, head_dim, nsplit, (const float*)p.part, u, l, m, p.c2,
                             scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention_chunk_stats combine launch");
  }
  return RA_OK;
}

int ra_merge_chunk_stats(int64_t rows, int head_dim, float* acc_u, float* acc_l, float* acc_m, const float* u,
                         const float* l, const float* m, void* stream) {
  g_err[0] = 0;
  if (rows < 0) return fail(RA_ERR_SHAPE, "rows=%lld", (long long)rows);
  if (head_dim < 1) return fail(RA_ERR_SHAPE, "head_dim=%d", head_dim);
  if (rows == 0) return RA_OK;
  if (!acc_u || !acc_l || !acc_m || !u || !l || !m) return fail(RA_ERR_NULL, "null statistics pointer");
  const bool vec4 = (head_dim % 4 == 0) && ((uintptr_t)acc_u % 16 == 0) && ((uintptr_t)u % 16 == 0);
  const int cols = vec4 ? head_dim / 4 : head_dim;
  int lpr = 1, sh = 0;
  while (lpr < cols && lpr < 64) {
    lpr <<= 1;
    ++sh;
  }
  const int64_t threads = rows * lpr;
  int64_t blocks = (threads + 255) / 256;
  const int64_t cap = 256 * 8 * 16;  // enough blocks to fill every CU several times over
  if (blocks > cap) blocks = cap;
  if (vec4)
    hipLaunchKernelGGL((merge_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, rows,
                       head_dim, lpr, sh, acc_u, acc_l, acc_m, u, l, m);
  else
    hipLaunchKernelGGL((merge_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, rows,
                       head_dim, lpr, sh, acc_u, acc_l, acc_m, u, l, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "merge_chunk_stats launch");
  return RA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Workspace of the allocation-free ring call: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends. Host code
// never uses the array's name as an address: the address on each device comes
// from hipGetSymbolAddress, looked up once per device with that device current.
namespace {
constexpr size_t kScratchBytes = RA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Address of `scratch` on the current device (looked up on the first call per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "ring_attention_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_UNSUPPORTED, "device index %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "ring_attention_noalloc: hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || (uintptr_t)ptr % 256 != 0)
      return fail(RA_ERR_HIP, "ring_attention_noalloc: scratch array at an unusable address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

// Block mask of a block-sparse call (see ra_ring_attention_block_sparse).
struct SparseSpec {
  const uint8_t* mask;  // device, [nqb][nkb]
  int64_t nqb, nkb;
  int64_t bq, bk;       // block sizes in positions (powers of two)
};

int log2_exact(int64_t x) {
  int l = 0;
  while (((int64_t)1 << l) < x) ++l;
  return ((int64_t)1 << l) == x ? l : -1;
}

// Rows of the block-sparse workspace beyond the ring call's own: the packed
// mask, and per query tile a tile count and a list of key tiles (sized for the
// general kernel's 128-row query tiles and 64-key tiles, the larger counts).
struct SparseLayout {
  int rw;              // words per packed mask row
  int64_t nqt, cap;    // query tiles and list row length provided for
  size_t bits, count, list, total;
};

SparseLayout sparse_layout(size_t base, int64_t q_len, int64_t total_keys, int64_t nqb, int64_t nkb) {
  SparseLayout L;
  L.rw = (int)((nkb + 31) / 32) + 1;
  L.nqt = (q_len + BM - 1) / BM;
  L.cap = (total_keys + BN - 1) / BN;
  L.bits = base;
  L.count = L.bits + align256(sizeof(uint32_t) * (size_t)nqb * (size_t)L.rw);
  L.list = L.count + align256(sizeof(int) * (size_t)(L.nqt > 0 ? L.nqt : 1));
  L.total = L.list + align256(sizeof(int) * (size_t)L.nqt * (size_t)(L.cap > 0 ? L.cap : 1));
  return L;
}

// True when every 32-row group of query rows (a wave of the pipelined kernel)
// lies in one query block of 2^lgq positions.
bool waves_in_one_qblock(const ra_q_segment* segs, int n, int lgq) {
  int64_t row = 0, wave_qb = -1;
  for (int s = 0; s < n; ++s) {
    const int64_t step = pos_step(segs[s].pos_stride);
    for (int64_t i = 0; i < segs[s].len; ++i, ++row) {
      const int64_t qb = (segs[s].global_offset + step * i) >> lgq;
      if ((row & 31) == 0)
        wave_qb = qb;
      else if (qb != wave_qb)
        return false;
    }
  }
  return true;
}

// The ring call. With use_scratch the workspace is the device's `scratch`
// array (workspace and workspace_bytes are ignored). With sp, the block mask
// restricts the visible keys as well.
int ring_attention_call(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                        const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks, int n_chunks,
                        int causal, float scale, void* workspace, size_t workspace_bytes, bool use_scratch,
                        const SparseSpec* sp, float* out, float* lse, void* stream) {
  g_err[0] = 0;
  int st = check_dims(dtype, batch, q_heads, kv_heads, head_dim);
  if (st) return st;
  if (n_q_segments < 1 || !q_segments) return fail(RA_ERR_NULL, "at least one query segment is required");
  if (n_chunks < 0 || (n_chunks > 0 && !chunks)) return fail(RA_ERR_NULL, "chunk array missing");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RA_ERR_SHAPE, "scale must be finite and > 0");
  const int64_t elem = dtype == RA_BF16 ? 2 : 4;
  int64_t lq = 0;
  for (int s = 0; s < n_q_segments; ++s) {
    const ra_q_segment& g = q_segments[s];
    if (g.len < 0) return fail(RA_ERR_SHAPE, "query segment %d: negative length", s);
    if (g.pos_stride < 0) return fail(RA_ERR_SHAPE, "query segment %d: negative pos_stride", s);
    if ((causal || sp) && g.len > 0 && !positions_fit(g.global_offset, g.len, pos_step(g.pos_stride)))
      return fail(RA_ERR_SHAPE, "query segment %d: positions outside [0, 2^31-1)", s);
    lq += g.len;
  }
  int64_t lk = 0;
  bool vec = true;
  for (int c = 0; c < n_chunks; ++c) {
    if ((st = check_chunk(chunks[c], c, head_dim))) return st;
    if ((st = check_row_stride(chunks[c], c))) return st;
    lk += chunks[c].len;
    vec = vec && chunk_vec_ok(chunks[c], head_dim, elem);
  }
  if (lk > kPosLimit) return fail(RA_ERR_UNSUPPORTED, "more than 2^31-2 keys in total");
  int lgq = 0, lgk = 0;
  if (sp) {
    lgq = log2_exact(sp->bq);
    lgk = log2_exact(sp->bk);
    if (lgq < 0 || lgk < 0 || lgq > 30 || lgk > 30)
      return fail(RA_ERR_SHAPE, "block sizes %lld x %lld must be powers of two up to 2^30", (long long)sp->bq,
                  (long long)sp->bk);
    if (sp->nqb < 1 || sp->nkb < 1 || sp->nqb > (1LL << 31) || sp->nkb > (1LL << 31))
      return fail(RA_ERR_SHAPE, "block mask of %lld x %lld blocks", (long long)sp->nqb, (long long)sp->nkb);
    for (int s = 0; s < n_q_segments; ++s) {
      const ra_q_segment& g = q_segments[s];
      if (g.len > 0 && (g.global_offset + pos_step(g.pos_stride) * (g.len - 1)) >> lgq >= sp->nqb)
        return fail(RA_ERR_SHAPE, "query segment %d reaches past the block mask's %lld query blocks", s,
                    (long long)sp->nqb);
    }
    for (int c = 0; c < n_chunks; ++c) {
      const ra_kv_chunk& ch = chunks[c];
      if (ch.len > 0 && (ch.global_offset + pos_step(ch.pos_stride) * (ch.len - 1)) >> lgk >= sp->nkb)
        return fail(RA_ERR_SHAPE, "chunk %d reaches past the block mask's %lld key blocks", c, (long long)sp->nkb);
    }
  }
  if (lq == 0 || batch == 0) return RA_OK;
  if (!q || !out) return fail(RA_ERR_NULL, "q and out must be non-null");
  if (sp && lk > 0 && !sp->mask) return fail(RA_ERR_NULL, "block mask is null");
  int kps = 1;
  const bool vecq = vec && vec_ok(q, head_dim, head_dim, elem);
  // block-sparse calls take the pipelined kernel when each wave's rows share a query block, the keys of a
  // tile are consecutive positions and a tile meets at most two key blocks; else the general kernel
  const bool pipe = sp ? (pipe_ok(dtype, head_dim, vecq, chunks, n_chunks, true, &kps) && kps == 1 &&
                          sp->bk >= pipe_tile(dp_of(head_dim)) && waves_in_one_qblock(q_segments, n_q_segments, lgq))
                       : pipe_ok(dtype, head_dim, vecq, chunks, n_chunks, causal != 0, &kps);
  if (sp) kps = 1;
  const int bm = pipe ? pipe_bm(kRingFull) : BM;
  const int64_t n_qt = (lq + bm - 1) / bm;
  const int64_t base_blocks = n_qt * q_heads * batch;
  const int nsplit = lk > 0 ? choose_nsplit(base_blocks, lk, pipe ? pipe_resident(kRingFull) : 2, causal ? 2 : 1) : 1;
  const int64_t nblocks = base_blocks * nsplit;
  if (nblocks > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid too large");
  const int64_t rows = (int64_t)batch * q_heads * lq;
  const size_t tbytes = table_bytes(n_chunks, n_q_segments);
  // the public size covers either kernel's key-range cut; the static scratch only needs the bytes this
  // call uses: its tables and the partials of the cut it runs with
  const size_t ring_bytes = ra_ring_workspace_bytes(batch, q_heads, head_dim, lq, lk, n_chunks, n_q_segments);
  const SparseLayout SL = sp ? sparse_layout(ring_bytes, lq, lk, sp->nqb, sp->nkb) : SparseLayout{};
  const size_t need = use_scratch ? tbytes + partial_bytes(nsplit, rows, head_dim) : (sp ? SL.total : ring_bytes);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(RA_ERR_WORKSPACE, "this share needs %zu bytes of workspace; the static scratch holds %zu", need,
                  kScratchBytes);
    if ((st = scratch_address(&workspace))) return st;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(RA_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, workspace_bytes);

  // Descriptor tables, written straight into the workspace on `stream`: the
  // non-empty chunks in list order, then the query segments.
  const size_t cbytes = align256(sizeof(ChunkDev) * (size_t)n_chunks);
  hipStream_t hs = (hipStream_t)stream;
  TableUpload up(workspace, hs);
  int nc = 0;
  int64_t start = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if (chunks[c].len == 0) continue;
    ChunkDev d = {};
    d.k = chunks[c].k;
    d.v = chunks[c].v;
    d.start = start;
    d.len = chunks[c].len;
    d.sb = chunks[c].stride_b;
    d.sh = chunks[c].stride_h;
    d.ss = chunks[c].stride_s;
    d.pos0 = (int32_t)chunks[c].global_offset;
    d.ps = (int32_t)pos_step(chunks[c].pos_stride);
    up.put(&d, sizeof(d));
    ++nc;
    start += chunks[c].len;
  }
  up.zero_to(cbytes);
  int64_t row0 = 0;
  for (int s = 0; s < n_q_segments; ++s) {
    QSegDev g = {};
    g.row0 = row0;
    g.len = q_segments[s].len;
    g.pos0 = q_segments[s].global_offset;
    g.ps = pos_step(q_segments[s].pos_stride);
    up.put(&g, sizeof(g));
    row0 += q_segments[s].len;
  }
  up.zero_to(tbytes);
  hipError_t e = up.finish();
  if (e != hipSuccess) return hip_fail(e, "ring_attention descriptor upload");

  Params p = {};
  p.q = q;
  p.o = out;
  p.l = lse;
  p.m = nullptr;
  p.part = nsplit > 1 ? (float*)((char*)workspace + tbytes) : nullptr;
  p.chunks = (const ChunkDev*)workspace;
  p.qsegs = (const QSegDev*)((char*)workspace + cbytes);
  p.Lq = lq;
  p.Lk = lk;
  p.n_chunks = nc > 0 ? nc : 1;  // with no keys the tile walk is empty and never reads the table
  p.n_qseg = n_q_segments;
  p.B = batch;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.d = head_dim;
  p.n_qt = (int)n_qt;
  p.nsplit = nsplit;
  p.vec = vec && vec_ok(q, head_dim, head_dim, elem);
  p.kps = kps;
  p.kinv = 1.0 / kps;
  p.scale = scale;
  p.c2 = scale * kLog2e;
  const bool mask = causal || lk % pipe_tile(dp_of(head_dim)) != 0;
  if (sp && lk > 0) {
    // pack the mask, then list each query tile's key tiles that hold an allowed pair
    char* ws = (char*)workspace;
    const int tb = pipe ? pipe_tile(dp_of(head_dim)) : BN;
    p.sp_bits = (const uint32_t*)(ws + SL.bits);
    p.sp_count = (const int*)(ws + SL.count);
    p.sp_list = (const int*)(ws + SL.list);
    p.sp_cap = (int)((lk + tb - 1) / tb);
    p.sp_rw = SL.rw;
    p.sp_lgq = lgq;
    p.sp_lgk = lgk;
    const int64_t nwords = sp->nqb * SL.rw;
    hipLaunchKernelGGL(sparse_bits_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, hs, sp->mask,
                       sp->nqb, sp->nkb, SL.rw, (uint32_t*)(ws + SL.bits));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "ring_attention_block_sparse mask packing launch");
    hipLaunchKernelGGL(sparse_plan_kernel, dim3((unsigned)n_qt), dim3(256), 0, hs, p.chunks, nc, p.qsegs,
                       n_q_segments, lq, lk, bm, tb, p.sp_bits, SL.rw, lgq, lgk, causal ? 1 : 0, p.sp_cap,
                       (int*)(ws + SL.list), (int*)(ws + SL.count));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "ring_attention_block_sparse plan launch");
  }
  timer_begin(hs);
  if (sp && lk > 0) {
    const int md = causal ? kRingCausal : kRingFull;
    e = md == kRingCausal ? launch_sparse_mode<kRingCausal>(dtype, dp_of(head_dim), pipe, p, (int)nblocks, hs)
                          : launch_sparse_mode<kRingFull>(dtype, dp_of(head_dim), pipe, p, (int)nblocks, hs);
  } else {
    e = launch(causal ? kRingCausal : kRingFull, dtype, dp_of(head_dim), p, pipe, mask, (int)nblocks, hs);
  }
  timer_end(hs);
  if (e != hipSuccess) return hip_fail(e, "ring_attention launch");
  if (nsplit > 1) {
    e = launch_combine<false>(rows, head_dim, nsplit, (const float*)p.part, out, lse, nullptr, p.c2, scale, hs);
    if (e != hipSuccess) return hip_fail(e, "ring_attention combine launch");
  }
  return RA_OK;
}

}  // namespace

extern "C" {

int ra_ring_attention(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                      const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks, int n_chunks,
                      int causal, float scale, void* workspace, size_t workspace_bytes, float* out, float* lse,
                      void* stream) {
  return ring_attention_call(dtype, batch, q_heads, kv_heads, head_dim, q, q_segments, n_q_segments, chunks,
                             n_chunks, causal, scale, workspace, workspace_bytes, false, nullptr, out, lse, stream);
}

size_t ra_block_sparse_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                                       int n_chunks, int n_q_segments, int64_t n_qblocks, int64_t n_kblocks) {
  if (q_len < 0) q_len = 0;
  if (total_keys < 0) total_keys = 0;
  if (n_qblocks < 1) n_qblocks = 1;
  if (n_kblocks < 1) n_kblocks = 1;
  const size_t base = ra_ring_workspace_bytes(batch, q_heads, head_dim, q_len, total_keys, n_chunks, n_q_segments);
  return sparse_layout(base, q_len, total_keys, n_qblocks, n_kblocks).total;
}

int ra_ring_attention_block_sparse(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                                   const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks,
                                   int n_chunks, int causal, float scale, const uint8_t* block_mask,
                                   int64_t n_qblocks, int64_t n_kblocks, int64_t block_q, int64_t block_k,
                                   void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream) {
  const SparseSpec sp = {block_mask, n_qblocks, n_kblocks, block_q, block_k};
  return ring_attention_call(dtype, batch, q_heads, kv_heads, head_dim, q, q_segments, n_q_segments, chunks,
                             n_chunks, causal, scale, workspace, workspace_bytes, false, &sp, out, lse, stream);
}

int ra_ring_attention_noalloc(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                              const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks,
                              int n_chunks, int causal, float scale, float* out, float* lse, void* stream) {
  return ring_attention_call(dtype, batch, q_heads, kv_heads, head_dim, q, q_segments, n_q_segments, chunks,
                             n_chunks, causal, scale, nullptr, 0, true, nullptr, out, lse, stream);
}

}  // extern "C"
