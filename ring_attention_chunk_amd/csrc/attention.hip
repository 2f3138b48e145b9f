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
//    owns 32 rows. The workgroup walks key tiles of BN = 64 keys in the order
//    of the concatenated chunk list, so tile boundaries never depend on how the
//    sequence was split into chunks: the result is bit-identical for any split.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l then holds one query (l % 32) and 16 of
//    the 32 keys of a block, so the row max and row sum are in-lane reductions
//    plus one exchange with lane l ^ 32. The probabilities stay in registers
//    and feed O^T = V^T P^T directly as the B operand (the key order inside a
//    16-key slice is permuted; V^T is stored in LDS with the same permutation).
//  * K tiles are staged row-major in LDS, V tiles transposed (d-major); both
//    are double-buffered, and the next tile is fetched from HBM into registers
//    while the current one is computed.
//  * With a causal mask, each tile is classified from global positions: tiles
//    whose first key lies after every query of the workgroup are skipped (and
//    whole chunks at once), tiles entirely in the past need no mask, the rest
//    compare positions per element (positions, never local indices).
//  * fp32 inputs take the same path with v_mfma_f32_32x32x2f32.
//  * The merge of two statistics is a separate bandwidth-bound kernel.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ring_attention_chunk.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int kPosNone = 0x7fffffff;          // position of a missing key: after everything
constexpr int kPosAll = 0x7ffffffe;           // query position that allows every real key
constexpr int kPosMin = -0x7fffffff - 1;      // query position of a missing row

enum Mode { kStats = 0, kRingFull = 1, kRingCausal = 2 };

// Chunk descriptor as the kernels read it (64 bytes).
struct ChunkDev {
  const void* k;
  const void* v;
  int64_t start;  // index of the chunk's first key in the concatenated list
  int64_t len;
  int64_t sb, sh, ss;
  int32_t pos0;  // global position of the first key
  int32_t pad;
};

struct QSegDev {
  int64_t row0;
  int64_t len;
  int64_t pos0;
};

struct Params {
  const void* q;
  float* o;    // out (ring) or u (stats)
  float* l;    // lse (ring, may be null) or l (stats)
  float* m;    // m (stats)
  const ChunkDev* chunks;
  const QSegDev* qsegs;
  ChunkDev one;  // the single chunk of the stats call
  int64_t Lq, Lk;
  int n_chunks, n_qseg;
  int B, Hq, Hkv, d;
  int n_qt;
  int vec;      // 16-byte loads allowed for q, k and v
  float scale;  // softmax scale
  float c2;     // scale * log2(e)
};

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

template <int MODE>
__device__ __forceinline__ ChunkDev chunk_at(const Params& p, int c) {
  if constexpr (MODE == kStats) {
    return p.one;
  } else {
    return p.chunks[c];
  }
}

// ---------------------------------------------------------------------------
// Element-type specific pieces: LDS layout, tile staging, MFMA fragments.

template <class T, int DP>
struct Ops;

// bf16: K row-major [BN][DP + 8], V transposed [DP][BN + 8] with the key order of
// each 16-key slice permuted (quads 1 and 2 swapped) to match the P fragments.
template <int DP>
struct Ops<__bf16, DP> {
  static constexpr int KP = DP + 8;
  static constexpr int VP = BN + 8;
  static constexpr int K_BYTES = BN * KP * 2;
  static constexpr int V_BYTES = DP * VP * 2;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES + BN * 4;
  static constexpr int CPR = DP / 8;                                   // 16-byte chunks per row
  static constexpr int NK = (BN * CPR + kThreads - 1) / kThreads;      // K items per thread
  static constexpr int NV = ((BN / 4) * CPR + kThreads - 1) / kThreads;  // V quad items per thread
  static constexpr int QF = DP / 16;

  struct Stage {
    u32x4 k[NK];
    u32x4 v[NV][4];
    int pos[NK];
  };
  struct QFrag {
    bf16x8 f[QF];
  };

  static __device__ __forceinline__ u32x4 load16(const __bf16* row, int c0, int d, bool vec) {
    if (vec) {
      if (c0 < d) return *(const u32x4*)(row + c0);
      return u32x4{0, 0, 0, 0};
    }
    const uint16_t* r = (const uint16_t*)row;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = (c0 + 2 * i < d) ? r[c0 + 2 * i] : 0u;
      uint32_t hi = (c0 + 2 * i + 1 < d) ? r[c0 + 2 * i + 1] : 0u;
      w[i] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }

  static __device__ __forceinline__ void load_q(const Params& p, const __bf16* qrow, bool valid,
                                                int h, QFrag& q) {
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      u32x4 x = valid ? load16(qrow, kk * 16 + h * 8, p.d, p.vec) : u32x4{0, 0, 0, 0};
      q.f[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Scores of one 32-key block of the tile (raw dot products), transposed.
  static __device__ __forceinline__ f32x16 qk(const char* buf, const QFrag& q, int kb, int lane) {
    const __bf16* Ks = (const __bf16*)buf;
    const __bf16* base = Ks + (kb * 32 + (lane & 31)) * KP + (lane >> 5) * 8;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      bf16x8 a = *(const bf16x8*)(base + kk * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.f[kk], acc, 0, 0, 0);
    }
    return acc;
  }

  // o[db] += V^T P^T over the tile, P taken from the (exponentiated) score blocks.
  static __device__ __forceinline__ void pv(const char* buf, const f32x16* s, f32x16* o, int lane) {
    const __bf16* Vs = (const __bf16*)(buf + K_BYTES);
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int t = 0; t < 8; ++t) pf[ks][t] = (__bf16)s[ks >> 1][(ks & 1) * 8 + t];
    }
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) {
      const __bf16* vrow = Vs + (db * 32 + (lane & 31)) * VP + (lane >> 5) * 8;
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        bf16x8 a = *(const bf16x8*)(vrow + ks * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ uint32_t pick(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
  }

  static __device__ __forceinline__ void store(char* buf, const Stage& st, int tid) {
    __bf16* Ks = (__bf16*)buf;
    __bf16* Vs = (__bf16*)(buf + K_BYTES);
    int* P = (int*)(buf + K_BYTES + V_BYTES);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      int item = tid + i * kThreads;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        int r = item / CPR, cc = item % CPR;
        *(u32x4*)(Ks + r * KP + cc * 8) = st.k[i];
        if (cc == 0) P[r] = st.pos[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int item = tid + i * kThreads;
      if (((BN / 4) * CPR) % kThreads == 0 || item < (BN / 4) * CPR) {
        int qd = item % (BN / 4), cc = item / (BN / 4);
        int qi = qd & 3;
        int pq = (qd & ~3) | (qi == 1 ? 2 : (qi == 2 ? 1 : qi));
        const u32x4* r = st.v[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dword w of each key row holds d = 2w (low half) and d = 2w + 1 (high half)
          uint32_t e0 = pick(r[1][w], r[0][w], 0x05040100u);
          uint32_t e1 = pick(r[3][w], r[2][w], 0x05040100u);
          uint32_t o0 = pick(r[1][w], r[0][w], 0x07060302u);
          uint32_t o1 = pick(r[3][w], r[2][w], 0x07060302u);
          *(u32x2*)(Vs + (cc * 8 + 2 * w) * VP + pq * 4) = u32x2{e0, e1};
          *(u32x2*)(Vs + (cc * 8 + 2 * w + 1) * VP + pq * 4) = u32x2{o0, o1};
        }
      }
    }
  }

  // Fetch tile rows [t0, t0 + BN) from HBM into registers.
  template <int MODE>
  static __device__ __forceinline__ void fetch(const Params& p, int64_t t0, int cursor, bool one_chunk,
                                               int b, int hk, int tid, Stage& st) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      int item = tid + i * kThreads;
      st.k[i] = u32x4{0, 0, 0, 0};
      st.pos[i] = kPosNone;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        int r = item / CPR, cc = item % CPR;
        const __bf16* kr;
        const __bf16* vr;
        int pos;
        if (row_src<MODE>(p, t0 + r, cursor, one_chunk, b, hk, kr, vr, pos)) {
          st.k[i] = load16(kr, cc * 8, p.d, p.vec);
          st.pos[i] = pos;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int item = tid + i * kThreads;
#pragma unroll
      for (int w = 0; w < 4; ++w) st.v[i][w] = u32x4{0, 0, 0, 0};
      if (((BN / 4) * CPR) % kThreads == 0 || item < (BN / 4) * CPR) {
        int qd = item % (BN / 4), cc = item / (BN / 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const __bf16* kr;
          const __bf16* vr;
          int pos;
          if (row_src<MODE>(p, t0 + qd * 4 + w, cursor, one_chunk, b, hk, kr, vr, pos))
            st.v[i][w] = load16(vr, cc * 8, p.d, p.vec);
        }
      }
    }
  }

  // Source rows of concatenated key index j (false if j is past the last key).
  template <int MODE>
  static __device__ __forceinline__ bool row_src(const Params& p, int64_t j, int cursor, bool one_chunk,
                                                 int b, int hk, const __bf16*& kr, const __bf16*& vr,
                                                 int& pos) {
    if (j >= p.Lk) return false;
    int c = cursor;
    if (!one_chunk) {
      while (c + 1 < p.n_chunks) {
        ChunkDev ch = chunk_at<MODE>(p, c);
        if (j < ch.start + ch.len) break;
        ++c;
      }
    }
    ChunkDev ch = chunk_at<MODE>(p, c);
    int64_t off = (int64_t)b * ch.sb + (int64_t)hk * ch.sh + (j - ch.start) * ch.ss;
    kr = (const __bf16*)ch.k + off;
    vr = (const __bf16*)ch.v + off;
    pos = ch.pos0 + (int)(j - ch.start);
    return true;
  }
};

// fp32: K and V both row-major [BN][DP + 4]; fragments for v_mfma_f32_32x32x2f32.
template <int DP>
struct Ops<float, DP> {
  static constexpr int KP = DP + 4;
  static constexpr int K_BYTES = BN * KP * 4;
  static constexpr int V_BYTES = BN * KP * 4;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES + BN * 4;
  static constexpr int CPR = DP / 4;
  static constexpr int NK = (BN * CPR + kThreads - 1) / kThreads;
  static constexpr int QF = DP / 2;

  struct Stage {
    u32x4 k[NK];
    u32x4 v[NK];
    int pos[NK];
  };
  struct QFrag {
    float f[QF];
  };

  static __device__ __forceinline__ u32x4 load16(const float* row, int c0, int d, bool vec) {
    if (vec) {
      if (c0 < d) return *(const u32x4*)(row + c0);
      return u32x4{0, 0, 0, 0};
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (c0 + i < d) ? __float_as_uint(row[c0 + i]) : 0u;
    return u32x4{w[0], w[1], w[2], w[3]};
  }

  static __device__ __forceinline__ void load_q(const Params& p, const float* qrow, bool valid, int h,
                                                QFrag& q) {
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      int c = 2 * kk + h;
      q.f[kk] = (valid && c < p.d) ? qrow[c] : 0.f;
    }
  }

  static __device__ __forceinline__ f32x16 qk(const char* buf, const QFrag& q, int kb, int lane) {
    const float* Ks = (const float*)buf;
    const float* base = Ks + (kb * 32 + (lane & 31)) * KP + (lane >> 5);
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < QF; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(base[2 * kk], q.f[kk], acc, 0, 0, 0);
    return acc;
  }

  static __device__ __forceinline__ void pv(const char* buf, const f32x16* s, f32x16* o, int lane) {
    const float* Vs = (const float*)(buf + K_BYTES);
    const int h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < DP / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * KP + db * 32 + (lane & 31)], s[kb][r],
                                                       o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store(char* buf, const Stage& st, int tid) {
    float* Ks = (float*)buf;
    float* Vs = (float*)(buf + K_BYTES);
    int* P = (int*)(buf + K_BYTES + V_BYTES);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      int item = tid + i * kThreads;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        int r = item / CPR, cc = item % CPR;
        *(u32x4*)(Ks + r * KP + cc * 4) = st.k[i];
        *(u32x4*)(Vs + r * KP + cc * 4) = st.v[i];
        if (cc == 0) P[r] = st.pos[i];
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ void fetch(const Params& p, int64_t t0, int cursor, bool one_chunk,
                                               int b, int hk, int tid, Stage& st) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      int item = tid + i * kThreads;
      st.k[i] = u32x4{0, 0, 0, 0};
      st.v[i] = u32x4{0, 0, 0, 0};
      st.pos[i] = kPosNone;
      if ((BN * CPR) % kThreads == 0 || item < BN * CPR) {
        int r = item / CPR, cc = item % CPR;
        const float* kr;
        const float* vr;
        int pos;
        if (row_src<MODE>(p, t0 + r, cursor, one_chunk, b, hk, kr, vr, pos)) {
          st.k[i] = load16(kr, cc * 4, p.d, p.vec);
          st.v[i] = load16(vr, cc * 4, p.d, p.vec);
          st.pos[i] = pos;
        }
      }
    }
  }

  template <int MODE>
  static __device__ __forceinline__ bool row_src(const Params& p, int64_t j, int cursor, bool one_chunk,
                                                 int b, int hk, const float*& kr, const float*& vr,
                                                 int& pos) {
    if (j >= p.Lk) return false;
    int c = cursor;
    if (!one_chunk) {
      while (c + 1 < p.n_chunks) {
        ChunkDev ch = chunk_at<MODE>(p, c);
        if (j < ch.start + ch.len) break;
        ++c;
      }
    }
    ChunkDev ch = chunk_at<MODE>(p, c);
    int64_t off = (int64_t)b * ch.sb + (int64_t)hk * ch.sh + (j - ch.start) * ch.ss;
    kr = (const float*)ch.k + off;
    vr = (const float*)ch.v + off;
    pos = ch.pos0 + (int)(j - ch.start);
    return true;
  }
};

// ---------------------------------------------------------------------------
// Tile walk (uniform across the workgroup): find the next tile at or after t
// that holds at least one key some query of the workgroup may see.

struct TileInfo {
  int64_t t;      // tile index (== ntiles when the walk is over)
  int cursor;     // chunk containing the tile's first key
  bool one_chunk; // all keys of the tile come from chunk `cursor`
  bool tail;      // the tile runs past the last key
  int kmin, kmax; // smallest / largest global key position in the tile
};

template <int MODE>
__device__ __forceinline__ TileInfo next_tile(const Params& p, int64_t t, int cursor, int64_t ntiles,
                                              int qmax) {
  TileInfo ti;
  while (t < ntiles) {
    const int64_t t0 = t * BN;
    const int64_t t1 = min(t0 + (int64_t)BN, p.Lk);
    // advance the cursor to the chunk holding key t0 (zero-length chunks are passed over)
    ChunkDev ch = chunk_at<MODE>(p, cursor);
    while (cursor + 1 < p.n_chunks && t0 >= ch.start + ch.len) {
      ++cursor;
      ch = chunk_at<MODE>(p, cursor);
    }
    int kmin = kPosNone, kmax = kPosMin;
    bool one = (t1 <= ch.start + ch.len);
    if (MODE == kRingCausal) {
      int c = cursor;
      ChunkDev cc = ch;
      while (true) {
        int64_t lo = max(t0, cc.start), hi = min(t1, cc.start + cc.len);
        if (lo < hi) {
          kmin = min(kmin, cc.pos0 + (int)(lo - cc.start));
          kmax = max(kmax, cc.pos0 + (int)(hi - 1 - cc.start));
        }
        if (c + 1 >= p.n_chunks || cc.start + cc.len >= t1) break;
        ++c;
        cc = chunk_at<MODE>(p, c);
      }
      if (kmin > qmax) {
        // nothing here is visible; if the whole chunk is in the future, jump past it
        if (one && ch.pos0 > qmax) {
          int64_t nt = (ch.start + ch.len) / BN;
          t = nt > t ? nt : t + 1;
        } else {
          ++t;
        }
        continue;
      }
    }
    ti.t = t;
    ti.cursor = cursor;
    ti.one_chunk = one;
    ti.tail = (t0 + BN > p.Lk);
    ti.kmin = kmin;
    ti.kmax = kmax;
    return ti;
  }
  ti.t = ntiles;
  ti.cursor = cursor;
  ti.one_chunk = true;
  ti.tail = false;
  ti.kmin = kPosNone;
  ti.kmax = kPosMin;
  return ti;
}

__device__ __forceinline__ int query_pos(const Params& p, int64_t row) {
  for (int s = 0; s < p.n_qseg; ++s) {
    QSegDev g = p.qsegs[s];
    if (row < g.row0 + g.len) return (int)(g.pos0 + (row - g.row0));
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

template <class T, int DP, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(Params p) {
  using O = Ops<T, DP>;
  __shared__ __attribute__((aligned(16))) char smem[2 * O::BUF_BYTES];
  __shared__ int qred[2 * kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;

  // Work decode. Blocks are dealt to the 8 XCDs round-robin; remap so that each
  // XCD gets a contiguous range of work items, and order items so that the
  // blocks sharing one key/value head (all q tiles of a head, and all query
  // heads of a GQA group) are adjacent and share that XCD's L2.
  int w = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) w = (w & 7) * (nwg >> 3) + (w >> 3);
  const int group = p.Hq / p.Hkv;
  const int g = w % group;
  w /= group;
  int qt = w % p.n_qt;
  w /= p.n_qt;
  const int hk = w % p.Hkv;
  const int b = w / p.Hkv;
  if (MODE == kRingCausal) qt = p.n_qt - 1 - qt;  // later queries see more keys: start them first
  const int hq = hk * group + g;

  const int64_t row = (int64_t)qt * BM + wave * 32 + (lane & 31);
  const bool valid = row < p.Lq;
  const int64_t qoff = (((int64_t)b * p.Hq + hq) * p.Lq + (valid ? row : 0)) * p.d;

  // Query positions and their bounds per wave and per workgroup.
  int qpos = kPosAll;
  int wqmin = kPosAll, wqmax = kPosAll, gqmax = kPosAll;
  if (MODE == kRingCausal) {
    qpos = valid ? query_pos(p, row) : kPosMin;
    wqmin = wave_min(valid ? qpos : kPosNone);
    wqmax = wave_max(valid ? qpos : kPosMin);
    if (lane == 0) {
      qred[wave] = wqmin;
      qred[kWaves + wave] = wqmax;
    }
    __syncthreads();
    gqmax = qred[kWaves];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) gqmax = max(gqmax, qred[kWaves + i]);
  }

  typename O::QFrag qf;
  O::load_q(p, (const T*)p.q + qoff, valid, h, qf);

  f32x16 o[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // running max of raw dot products <q, k>
  float l_run = 0.f;        // this lane's share of the running denominator

  const int64_t ntiles = (p.Lk + BN - 1) / BN;
  typename O::Stage st;
  TileInfo cur = next_tile<MODE>(p, 0, 0, ntiles, gqmax);
  if (cur.t < ntiles) {
    O::template fetch<MODE>(p, cur.t * BN, cur.cursor, cur.one_chunk, b, hk, tid, st);
    O::store(smem, st, tid);
  }
  __syncthreads();
  int buf = 0;
  while (cur.t < ntiles) {
    TileInfo nxt = next_tile<MODE>(p, cur.t + 1, cur.cursor, ntiles, gqmax);
    if (nxt.t < ntiles) O::template fetch<MODE>(p, nxt.t * BN, nxt.cursor, nxt.one_chunk, b, hk, tid, st);

    // Per-wave view of the tile: nothing visible, everything visible, or mixed.
    bool skip = false, masked = cur.tail;
    if (MODE == kRingCausal) {
      skip = cur.kmin > wqmax;
      masked = masked || cur.kmax > wqmin;
    }
    if (!skip) {
      const char* tb = smem + buf * O::BUF_BYTES;
      f32x16 s[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) s[kb] = O::qk(tb, qf, kb, lane);
      if (masked) {
        const int* kp = (const int*)(tb + O::K_BYTES + O::V_BYTES);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (kp[key] > qpos) s[kb][r] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = fmaxf(mt, wave_xor32(mt));
      const float mnew = fmaxf(m_run, mt);
      const float ms = (mnew == -INFINITY) ? 0.f : mnew * p.c2;
      const float alpha = __builtin_amdgcn_exp2f(m_run * p.c2 - ms);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], p.c2, -ms));
          s[kb][r] = e;
          rs += e;
        }
      l_run = fmaf(l_run, alpha, rs);
      m_run = mnew;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DP / 32; ++db) o[db] *= alpha;
      }
      O::pv(tb, s, o, lane);
    }

    if (nxt.t < ntiles) O::store(smem + (buf ^ 1) * O::BUF_BYTES, st, tid);
    __syncthreads();
    buf ^= 1;
    cur = nxt;
  }

  // Epilogue: combine the two half-waves' denominators, then write.
  const float l = l_run + wave_xor32(l_run);
  if (!valid) return;
  float* orow = p.o + qoff;
  float inv = 1.f;
  if (MODE != kStats) inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int db = 0; db < DP / 32; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int c0 = db * 32 + 8 * gi + 4 * h;
      f32x4 v = {o[db][4 * gi] * inv, o[db][4 * gi + 1] * inv, o[db][4 * gi + 2] * inv,
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
    const int64_t ri = ((int64_t)b * p.Hq + hq) * p.Lq + row;
    const float m_out = (m_run == -INFINITY) ? -INFINITY : m_run * p.scale;
    if (MODE == kStats) {
      p.l[ri] = l;
      p.m[ri] = m_out;
    } else if (p.l != nullptr) {
      p.l[ri] = (l > 0.f) ? m_out + logf(l) : -INFINITY;
    }
  }
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
    if (VEC4) {
      const int n4 = d >> 2;
      f32x4* pa = (f32x4*)(au + r * d);
      const f32x4* pb = (const f32x4*)(bu + r * d);
      for (int c = sub; c < n4; c += lpr) {
        f32x4 x = pa[c], y = pb[c];
        pa[c] = x * fa + y * fb;
      }
    } else {
      float* pa = au + r * d;
      const float* pb = bu + r * d;
      for (int c = sub; c < d; c += lpr) pa[c] = pa[c] * fa + pb[c] * fb;
    }
    if (sub == 0) {
      am[r] = mx;
      al[r] = la * fa + lb * fb;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, descriptor tables, dispatch.

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kPosLimit = 0x7ffffffeLL;

int check_dims(int dtype, int batch, int q_heads, int kv_heads, int head_dim) {
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0)
    return fail(RA_ERR_SHAPE, "batch=%d q_heads=%d kv_heads=%d", batch, q_heads, kv_heads);
  if (q_heads % kv_heads != 0)
    return fail(RA_ERR_SHAPE, "q_heads=%d is not a multiple of kv_heads=%d", q_heads, kv_heads);
  if (head_dim < 1 || head_dim > 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim=%d outside 1..128", head_dim);
  return RA_OK;
}

int check_chunk(const ra_kv_chunk& c, int idx, int batch, int kv_heads, int head_dim, int64_t elem) {
  if (c.len < 0) return fail(RA_ERR_SHAPE, "chunk %d: negative length", idx);
  if (c.len == 0) return RA_OK;
  if (!c.k || !c.v) return fail(RA_ERR_NULL, "chunk %d: null k or v", idx);
  if (c.global_offset < 0 || c.global_offset + c.len - 1 > kPosLimit)
    return fail(RA_ERR_SHAPE, "chunk %d: positions [%lld, %lld) outside [0, 2^31-1)", idx,
                (long long)c.global_offset, (long long)(c.global_offset + c.len));
  if (c.stride_s < head_dim || c.stride_b < 0 || c.stride_h < 0)
    return fail(RA_ERR_SHAPE, "chunk %d: strides b=%lld h=%lld s=%lld invalid for head_dim %d", idx,
                (long long)c.stride_b, (long long)c.stride_h, (long long)c.stride_s, head_dim);
  (void)batch;
  (void)kv_heads;
  (void)elem;
  return RA_OK;
}

bool vec_ok(const void* p, int64_t stride, int head_dim, int64_t elem) {
  const int64_t per16 = 16 / elem;
  return ((uintptr_t)p % 16 == 0) && stride % per16 == 0 && head_dim % per16 == 0;
}

int dp_of(int head_dim) { return head_dim <= 32 ? 32 : (head_dim <= 64 ? 64 : 128); }

template <class T, int DP, int MODE>
hipError_t launch_t(const Params& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((attention_kernel<T, DP, MODE>), dim3(nblocks), dim3(kThreads), 0, s, p);
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

hipError_t launch(int mode, int dtype, int dp, const Params& p, int nblocks, hipStream_t s) {
  if (mode == kStats) return launch_mode<kStats>(dtype, dp, p, nblocks, s);
  if (mode == kRingFull) return launch_mode<kRingFull>(dtype, dp, p, nblocks, s);
  return launch_mode<kRingCausal>(dtype, dp, p, nblocks, s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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

size_t ra_ring_workspace_bytes(int n_chunks, int n_q_segments) {
  if (n_chunks < 0) n_chunks = 0;
  if (n_q_segments < 0) n_q_segments = 0;
  return align256(sizeof(ChunkDev) * (size_t)n_chunks) + align256(sizeof(QSegDev) * (size_t)n_q_segments) + 256;
}

int ra_attention_chunk_stats(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                             const void* q, int64_t q_len, const ra_kv_chunk* chunk, float scale,
                             float* u, float* l, float* m, void* stream) {
  g_err[0] = 0;
  int st = check_dims(dtype, batch, q_heads, kv_heads, head_dim);
  if (st) return st;
  if (!chunk) return fail(RA_ERR_NULL, "chunk descriptor is null");
  if (q_len < 0) return fail(RA_ERR_SHAPE, "q_len=%lld", (long long)q_len);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RA_ERR_SHAPE, "scale must be finite and > 0");
  const int64_t elem = dtype == RA_BF16 ? 2 : 4;
  if ((st = check_chunk(*chunk, 0, batch, kv_heads, head_dim, elem))) return st;
  if (q_len == 0 || batch == 0) return RA_OK;
  if (!q || !u || !l || !m) return fail(RA_ERR_NULL, "q, u, l and m must be non-null");
  if (chunk->len > kPosLimit) return fail(RA_ERR_UNSUPPORTED, "chunk longer than 2^31-2 keys");
  const int64_t n_qt = (q_len + BM - 1) / BM;
  const int64_t nblocks = n_qt * q_heads * batch;
  if (nblocks > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid too large");

  Params p = {};
  p.q = q;
  p.o = u;
  p.l = l;
  p.m = m;
  p.one.k = chunk->k;
  p.one.v = chunk->v;
  p.one.start = 0;
  p.one.len = chunk->len;
  p.one.sb = chunk->stride_b;
  p.one.sh = chunk->stride_h;
  p.one.ss = chunk->stride_s;
  p.one.pos0 = 0;
  p.Lq = q_len;
  p.Lk = chunk->len;
  p.n_chunks = 1;
  p.n_qseg = 0;
  p.B = batch;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.d = head_dim;
  p.n_qt = (int)n_qt;
  p.vec = vec_ok(q, head_dim, head_dim, elem) &&
          (chunk->len == 0 || (vec_ok(chunk->k, chunk->stride_s, head_dim, elem) &&
                               vec_ok(chunk->v, chunk->stride_s, head_dim, elem) &&
                               chunk->stride_b % (16 / elem) == 0 && chunk->stride_h % (16 / elem) == 0));
  p.scale = scale;
  p.c2 = scale * 1.4426950408889634f;
  hipError_t e = launch(kStats, dtype, dp_of(head_dim), p, (int)nblocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention_chunk_stats launch");
  return RA_OK;
}

int ra_merge_chunk_stats(int64_t rows, int head_dim, float* acc_u, float* acc_l, float* acc_m,
                         const float* u, const float* l, const float* m, void* stream) {
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

int ra_ring_attention(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                      const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks,
                      int n_chunks, int causal, float scale, void* workspace, size_t workspace_bytes,
                      float* out, float* lse, void* stream) {
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
    if (causal && g.len > 0 && (g.global_offset < 0 || g.global_offset + g.len - 1 > kPosLimit))
      return fail(RA_ERR_SHAPE, "query segment %d: positions outside [0, 2^31-1)", s);
    lq += g.len;
  }
  int64_t lk = 0;
  bool vec = true;
  for (int c = 0; c < n_chunks; ++c) {
    if ((st = check_chunk(chunks[c], c, batch, kv_heads, head_dim, elem))) return st;
    lk += chunks[c].len;
    if (chunks[c].len > 0)
      vec = vec && vec_ok(chunks[c].k, chunks[c].stride_s, head_dim, elem) &&
            vec_ok(chunks[c].v, chunks[c].stride_s, head_dim, elem) &&
            chunks[c].stride_b % (16 / elem) == 0 && chunks[c].stride_h % (16 / elem) == 0;
  }
  if (lk > kPosLimit) return fail(RA_ERR_UNSUPPORTED, "more than 2^31-2 keys in total");
  if (lq == 0 || batch == 0) return RA_OK;
  if (!q || !out) return fail(RA_ERR_NULL, "q and out must be non-null");
  const size_t need = ra_ring_workspace_bytes(n_chunks, n_q_segments);
  if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(RA_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  const int64_t n_qt = (lq + BM - 1) / BM;
  const int64_t nblocks = n_qt * q_heads * batch;
  if (nblocks > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid too large");

  // Descriptor tables: chunks (non-empty ones only; order kept) then query segments.
  const size_t cbytes = align256(sizeof(ChunkDev) * (size_t)n_chunks);
  const size_t qbytes = align256(sizeof(QSegDev) * (size_t)n_q_segments);
  char* host = (char*)calloc(1, cbytes + qbytes);
  if (!host) return fail(RA_ERR_UNSUPPORTED, "host allocation failed");
  ChunkDev* hc = (ChunkDev*)host;
  QSegDev* hq = (QSegDev*)(host + cbytes);
  int nc = 0;
  int64_t start = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if (chunks[c].len == 0) continue;
    ChunkDev& d = hc[nc++];
    d.k = chunks[c].k;
    d.v = chunks[c].v;
    d.start = start;
    d.len = chunks[c].len;
    d.sb = chunks[c].stride_b;
    d.sh = chunks[c].stride_h;
    d.ss = chunks[c].stride_s;
    d.pos0 = (int32_t)chunks[c].global_offset;
    start += chunks[c].len;
  }
  int64_t row0 = 0;
  for (int s = 0; s < n_q_segments; ++s) {
    hq[s].row0 = row0;
    hq[s].len = q_segments[s].len;
    hq[s].pos0 = q_segments[s].global_offset;
    row0 += q_segments[s].len;
  }
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(workspace, host, cbytes + qbytes, hipMemcpyHostToDevice, hs);
  free(host);
  if (e != hipSuccess) return hip_fail(e, "ring_attention descriptor copy");

  Params p = {};
  p.q = q;
  p.o = out;
  p.l = lse;
  p.m = nullptr;
  p.chunks = (const ChunkDev*)workspace;
  p.qsegs = (const QSegDev*)((char*)workspace + cbytes);
  p.Lq = lq;
  p.Lk = lk;
  p.n_chunks = nc > 0 ? nc : 1;
  p.n_qseg = n_q_segments;
  p.B = batch;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.d = head_dim;
  p.n_qt = (int)n_qt;
  p.vec = vec && vec_ok(q, head_dim, head_dim, elem);
  p.scale = scale;
  p.c2 = scale * 1.4426950408889634f;
  if (nc == 0) {
    // no keys at all: the tile walk is empty, every row ends with l = 0
    p.chunks = (const ChunkDev*)workspace;
  }
  e = launch(causal ? kRingCausal : kRingFull, dtype, dp_of(head_dim), p, (int)nblocks, hs);
  if (e != hipSuccess) return hip_fail(e, "ring_attention launch");
  return RA_OK;
}

}  // extern "C"
