// backward.hip -- gradients of ring attention for one device's share (gfx950).
//
// What is computed ("Ring Attention: Distributed Reads with Online Softmax",
// section "Backward must aggregate shared dependencies"): the local queries
// contribute gradients to the keys and values of every chunk they attend to;
// the contributions to one key are summed (over all local queries and, with
// GQA, over the query heads sharing its key/value head) and handed back per
// chunk, to be returned to the chunk's owner. Probability tiles are recomputed
// from the forward's log-sum-exp with the same scale and the same global-
// position causal mask as the forward pass. With p = exp(s - lse) and
// delta_i = <dO_i, out_i>:
//   dV_j = sum_i p_ij dO_i,   dS_ij = p_ij (<dO_i, v_j> - delta_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
//
// Mapping onto the chip
// ---------------------
//  * delta_kernel: one pass over dO and out (HBM-bound).
//  * dkdv_kernel: a workgroup owns 128 keys of one (batch, kv head), 32 per
//    wave, and walks every query row of every query head of its group in
//    blocks of 32. K and V stay in registers as MFMA B operands; each query
//    block (Q, dO, lse, delta, positions) is staged once in a ring of LDS
//    slots for the four waves, its global loads issued two blocks ahead, and
//    the work is software-pipelined across blocks (see the kernel). S = Q K^T and dP = dO V^T
//    put one key per lane and 16 queries in its registers; those registers,
//    rounded to bf16, are directly the B operand of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands are read transposed from the row-major
//    tiles (ds_read_b64_tr_b16) in the same (permuted) query order.
//  * dq_kernel: a workgroup owns 128 query rows of one (batch, head), 32 per
//    wave, and walks the keys in tiles of 32. Q and dO stay in registers;
//    S^T = K Q^T and dP^T = V dO^T put one query per lane; dQ^T += K^T dS^T.
//  * Both gradient kernels give every output row to exactly one lane and sum
//    in a fixed order: no atomics, bit-reproducible results.
//  * Query blocks that lie before every key of a workgroup, and key tiles that
//    lie after every query of a workgroup, are skipped (causal).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "host_common.h"
#include "ring_attention_chunk.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kRows = 32;                    // rows per MFMA block (keys or queries)
constexpr int kGroupRows = kRows * kBwdWaves;  // rows per workgroup
constexpr int kPosMax = 0x7fffffff;          // position of a missing key: after everything
constexpr int kPosAllQ = 0x7ffffffe;         // query position that sees every real key
constexpr int kPosMinQ = -0x7fffffff - 1;    // position of a missing query row: sees nothing
constexpr float kLog2e = 1.4426950408889634f;

// Workgroups are dealt to the 8 XCDs round-robin; when the grid is a multiple of
// 8, renumber them so that each XCD takes one contiguous range of work items and
// the items running together on an XCD share that XCD's L2.
__device__ __forceinline__ int xcd_item(int blk, int nwg) {
  return (nwg & 7) == 0 ? (blk & 7) * (nwg >> 3) + (blk >> 3) : blk;
}

struct BwdChunk {
  const void* k;
  const void* v;
  int64_t start;  // index of the chunk's first key in the concatenated list
  int64_t len;
  int64_t sb, sh, ss;
  int32_t pos0, ps;
};

struct BwdParams {
  const __bf16* q;     // [B, Hq, Lq, d]
  const __bf16* dout;  // [B, Hq, Lq, d]
  const float* out;    // [B, Hq, Lq, d]
  const float* lse;    // [B, Hq, Lq]
  float* delta;        // [B, Hq, Lq] (workspace)
  const int* qpos;     // [Lq] query positions (kPosAllQ when not causal)
  const int* kpos;     // [Lk] key positions in list order
  const int* qblk;     // [ceil(Lq / 32)][2] smallest and largest query position of each 32-row block
  const int* ktile;    // [ceil(Lk / 32)][2] smallest and largest key position of each 32-key tile
  const BwdChunk* chunks;
  float* dq;           // [B, Hq, Lq, d]
  float* dk;           // [B, Hkv, Lk, d]
  float* dv;           // [B, Hkv, Lk, d]
  int64_t Lq, Lk;
  int n_chunks;
  int B, Hq, Hkv, d;
  int causal;
  float scale;
  float c2;  // scale * log2(e)
  int dq_split;    // key-tile ranges of the dQ kernel (1: dQ written directly)
  float* dq_part;  // [dq_split][B * Hq * Lq][d] unscaled partial dQ when dq_split > 1 (workspace)
};

// Chunk descriptors read through the constant address space: with an index that is the same for every
// lane these become scalar loads.
typedef const __attribute__((address_space(4))) BwdChunk* cchunk_ptr;
__device__ __forceinline__ BwdChunk chunk_at(const BwdChunk* chunks, int i) {
  const cchunk_ptr c = (cchunk_ptr)chunks + i;
  BwdChunk r;
  r.k = c->k;
  r.v = c->v;
  r.start = c->start;
  r.len = c->len;
  r.sb = c->sb;
  r.sh = c->sh;
  r.ss = c->ss;
  r.pos0 = c->pos0;
  r.ps = c->ps;
  return r;
}
typedef const __attribute__((address_space(4))) int* cint_ptr;
__device__ __forceinline__ int cload(const int* p) { return *(cint_ptr)p; }

// Per-lane reads of the chunk table and of key rows through the global address
// space. Through a generic pointer they would be flat loads, which count on the
// LDS wait counter as well: one in a loop makes the compiler wait for every
// outstanding LDS read (lgkmcnt(0)) wherever the loop waits for one.
typedef const __attribute__((address_space(1))) BwdChunk* gchunk_ptr;
typedef const __attribute__((address_space(1))) u32x4* gu32x4_ptr;
__device__ __forceinline__ u32x4 gload16(const void* ptr) { return *(gu32x4_ptr)ptr; }

// Row address of key j (chunk `c` holds it); the cursor only moves forward.
__device__ __forceinline__ int64_t key_offset(const BwdParams& p, int64_t j, int b, int hk, int& c) {
  const gchunk_ptr chunks = (gchunk_ptr)p.chunks;
  while (c + 1 < p.n_chunks && j >= chunks[c].start + chunks[c].len) ++c;
  return (int64_t)b * chunks[c].sb + (int64_t)hk * chunks[c].sh + (j - chunks[c].start) * chunks[c].ss;
}
// Key pointer of chunk c.
__device__ __forceinline__ const __bf16* chunk_k(const BwdParams& p, int c) {
  return (const __bf16*)((gchunk_ptr)p.chunks)[c].k;
}
__device__ __forceinline__ const __bf16* chunk_v(const BwdParams& p, int c) {
  return (const __bf16*)((gchunk_ptr)p.chunks)[c].v;
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& x, int t) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[8 * t + i];
  return r;
}

// ---------------------------------------------------------------------------
// delta_i = <dO_i, out_i>: DP/8 lanes per row, 16-byte loads of dO.

__global__ __launch_bounds__(256) void delta_kernel(int64_t rows, int d, int lpr, int lpr_shift,
                                                    const __bf16* __restrict__ dout, const float* __restrict__ out,
                                                    float* __restrict__ delta) {
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> lpr_shift;
  const int sub = threadIdx.x & (lpr - 1);
  float acc = 0.f;
  if (r < rows) {
    for (int c = sub * 8; c < d; c += lpr * 8) {
      const u32x4 raw = *(const u32x4*)(dout + r * d + c);
      const bf16x8 g = __builtin_bit_cast(bf16x8, raw);
      const f32x4 o0 = *(const f32x4*)(out + r * d + c);
      const f32x4 o1 = *(const f32x4*)(out + r * d + c + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf((float)g[i], o0[i], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf((float)g[4 + i], o1[i], acc);
    }
  }
  for (int o = lpr >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (r < rows && sub == 0) delta[r] = acc;
}

// ---------------------------------------------------------------------------
// 32-row blocks of a [rows, d] bf16 tensor in LDS, row-major without padding,
// the 16-byte pieces of each row permuted by an XOR swizzle (piece c of row r
// sits at position c ^ swz(r)) so that both operand reads hit distinct banks:
// 16 consecutive rows at one piece (row reads) and 4 consecutive rows x 4
// consecutive pieces (transposing reads). Blocks go HBM -> registers (issued
// ahead, so the loads run under earlier matrix work) -> LDS.

template <int DP>
struct Tile {
  static constexpr int RS = DP;                          // row stride (elements)
  static constexpr int ROWB = 2 * DP;                    // row stride (bytes)
  static constexpr int NS = DP / 16;                     // k-steps over head_dim
  static constexpr int NB = DP / 32;                     // 32-column blocks
  static constexpr int PIECES = kRows * DP / 8;          // 16-byte pieces per block
  static constexpr int PER = (PIECES + kBwdThreads - 1) / kBwdThreads;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

  static __device__ __forceinline__ int swz(int r) {
    if constexpr (DP == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (DP == 64) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }

  // piece k of this thread: row and 8-column group; false past the block
  static __device__ __forceinline__ bool piece(int tid, int k, int& r, int& c8) {
    const int pc = tid + k * kBwdThreads;
    r = pc / (DP / 8);
    c8 = pc % (DP / 8);
    return PIECES % kBwdThreads == 0 || pc < PIECES;
  }

  static __device__ __forceinline__ void put(__bf16* rm, int tid, const u32x4* regs) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int r, c8;
      if (piece(tid, k, r, c8)) *(u32x4*)(rm + r * RS + ((c8 ^ swz(r)) << 3)) = regs[k];
    }
  }

  // Per-lane LDS byte offsets of the operands, fixed for the whole kernel.
  //  row[s]: A operand of a 32x32x16 MFMA, row lane % 32 of the block, k = 16 s + 8 h .. +7.
  //  col[db][hh]: half hh of the A operand holding the block transposed: row db * 32 + lane % 32 of
  //  the transpose (a column of the block), and k slots in the order of an MFMA output's registers
  //  8t .. 8t+7, i.e. block rows 16t + 4h .. +3 (hh = 0), then 16t + 8 + 4h .. +3 (hh = 1); add 16t
  //  rows, which leave the swizzle unchanged. Each half is one ds_read_b64_tr_b16: lane j of a 16-lane
  //  group addresses block row base + j / 4, columns c0 + 4 (j % 4) .. +3, and lane i of the group
  //  receives column c0 + i of block rows base .. base + 3.
  struct Lanes {
    int row[NS];
    int col[NB][2];
  };
  static __device__ __forceinline__ Lanes lanes(int lane) {
    Lanes L;
    const int r = lane & 31, h = lane >> 5, j = lane & 15;
#pragma unroll
    for (int s = 0; s < NS; ++s) L.row[s] = r * ROWB + (((2 * s + h) ^ swz(r)) << 4);
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 4 * h + 8 * hh + (j >> 2);
        const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
        L.col[db][hh] = row * ROWB + (((col >> 3) ^ swz(row)) << 4) + 2 * (col & 7);
      }
    return L;
  }

  static __device__ __forceinline__ bf16x8 rows_frag(const __bf16* rm, const Lanes& L, int s) {
    return *(const bf16x8*)((const char*)rm + L.row[s]);
  }

  static __device__ __forceinline__ bf16x8 cols_frag(const __bf16* rm, const Lanes& L, int db, int t) {
    const char* a = (const char*)rm + t * 16 * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(a + L.col[db][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(a + L.col[db][1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Output register r of a 32x32 MFMA block sits at row 8 (r / 4) + 4 h + r % 4.
__device__ __forceinline__ int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// dK and dV of 128 keys per workgroup, software-pipelined over query blocks.
//
// The query blocks the workgroup visits pass through a ring of four LDS slots
// (Q, dO, lse, delta and positions of 32 rows each). Iteration i of the walk
// first writes block i + 2, loaded into registers during the previous
// iteration, into its slot and issues the global loads of block i + 3. Then
// one phase of fixed slots: each slot issues one MFMA, alternately a product
// of dV/dK for block i - 1 (from the bf16 P and dS the previous phase made)
// and one of S/dP for block i + 1, and the vector units turn S(i) and dP(i),
// finished in the previous phase, into the bf16 P(i) and dS(i) of the next
// phase. No vector instruction of a phase waits on an MFMA of that phase, and
// the matrix pipe always has independent work queued. One barrier closes the
// iteration: it publishes block i + 2 and frees the slot of block i - 1.
// Every accumulator sums its products in the same order as a plain loop over
// the blocks would.

template <int DP>
struct QBlock {
  __bf16 q[kRows * Tile<DP>::RS];
  __bf16 g[kRows * Tile<DP>::RS];
  float lse2[kRows];  // lse * log2(e) (0 for rows that see nothing)
  float del[kRows];
  int qp[kRows];
};
constexpr int kRing = 4;

// Slot of a phase of nmf slots in which register r of S and dP is turned into P and dS.
constexpr int vec_slot(int r, int nmf) {
  int sl = 0;
  while (16 * (sl + 1) / nmf <= r) ++sl;
  return sl;
}

template <int V>
struct BIntC {
  static constexpr int value = V;
};

__device__ __forceinline__ bf16x8 words_bf16x8(const uint32_t (&w)[4]) {
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// Two workgroups per CU where the registers allow (head_dim <= 64): the waves of
// one then hide the barrier and LDS latency of the other.
constexpr int dkdv_resident(int dp) { return dp <= 64 ? 2 : 1; }

template <int DP, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, dkdv_resident(DP)) void dkdv_kernel(BwdParams p) {
  using T = Tile<DP>;
  constexpr int NS = DP / 16;           // k-steps over head_dim
  constexpr int NB = DP / 32;           // 32-row blocks of head_dim
  constexpr int PER = T::PER;
  constexpr int NMF = 4 * NB + 2 * NS;  // MFMAs per phase: dV/dK of one block and S/dP of another
  constexpr int kRA = DP >= 128 ? 4 : 2;  // slots between an operand read and its MFMA
  __shared__ __attribute__((aligned(16))) QBlock<DP> ring[kRing];
  __shared__ int kmin_red[2 * kBwdWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const typename T::Lanes LL = T::lanes(lane);
  const int n_kt = (int)((p.Lk + kGroupRows - 1) / kGroupRows);
  // causal: the renumbering below measured +10-40% on causal shares (unequal work per item)
  // and -1% on the non-causal long GQA share, which keeps the plain order
  const int item = CAUSAL ? xcd_item(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int kt = item % n_kt;
  const int bh = item / n_kt;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int group = p.Hq / p.Hkv;

  // this lane's key: its K and V rows as B operands, and its position
  const int64_t j = (int64_t)kt * kGroupRows + wave * kRows + (lane & 31);
  const bool kvalid = j < p.Lk;
  bf16x8 kf[NS], vf[NS];
  int kp = kPosMax;
  {
    int c = 0;
    const int64_t off = kvalid ? key_offset(p, j, b, hk, c) : 0;
    const __bf16* kr = chunk_k(p, c) + off;
    const __bf16* vr = chunk_v(p, c) + off;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = 16 * s + 8 * h;
      u32x4 kraw = {0u, 0u, 0u, 0u}, vraw = {0u, 0u, 0u, 0u};
      if (kvalid && col < p.d) {
        kraw = gload16(kr + col);
        vraw = gload16(vr + col);
      }
      kf[s] = __builtin_bit_cast(bf16x8, kraw);
      vf[s] = __builtin_bit_cast(bf16x8, vraw);
    }
    if (kvalid) kp = p.kpos[j];
  }
  // smallest and largest key position of the workgroup: query blocks entirely before the smallest
  // see nothing here, and blocks entirely at or after the largest see everything (no mask)
  int wk = kp, wx = kvalid ? kp : kPosMinQ;
  for (int o = 32; o > 0; o >>= 1) {
    wk = min(wk, __shfl_xor(wk, o));
    wx = max(wx, __shfl_xor(wx, o));
  }
  if (lane == 0) {
    kmin_red[wave] = wk;
    kmin_red[kBwdWaves + wave] = wx;
  }
  __syncthreads();
  int kmin = kmin_red[0], kmax = kmin_red[kBwdWaves];
  for (int w = 1; w < kBwdWaves; ++w) {
    kmin = min(kmin, kmin_red[w]);
    kmax = max(kmax, kmin_red[kBwdWaves + w]);
  }

  f32x16 dkT[NB], dvT[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    dkT[i] = f32x16{};
    dvT[i] = f32x16{};
  }

  // walk (query head of the group, 32-row block) in order, skipping blocks that see none of our keys;
  // never called again once it has returned false
  const int n_qb = (int)((p.Lq + kRows - 1) / kRows);
  auto advance = [&](int& g, int& qb) {
    while (true) {
      if (++qb >= n_qb) {
        qb = 0;
        if (++g >= group) return false;
      }
      if (!CAUSAL || cload(p.qblk + 2 * qb + 1) >= kmin) return true;
    }
  };
  u32x4 pq[PER], pg[PER];
  float pl = 0.f, pd = 0.f;
  int pp = kPosMinQ;
  auto fetch = [&](int g, int qb) {
    const int64_t rowbase = ((int64_t)b * p.Hq + hk * group + g) * p.Lq;
    const int64_t r0 = (int64_t)qb * kRows;
    const int64_t nrows = min((int64_t)kRows, p.Lq - r0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int r, c8;
      pq[k] = u32x4{0u, 0u, 0u, 0u};
      pg[k] = u32x4{0u, 0u, 0u, 0u};
      if (T::piece(tid, k, r, c8) && r < nrows && c8 * 8 < p.d) {
        pq[k] = *(const u32x4*)(p.q + (rowbase + r0 + r) * p.d + c8 * 8);
        pg[k] = *(const u32x4*)(p.dout + (rowbase + r0 + r) * p.d + c8 * 8);
      }
    }
    if (tid < kRows) {
      const bool v = tid < nrows;
      pl = v ? p.lse[rowbase + r0 + tid] : 0.f;
      pd = v ? p.delta[rowbase + r0 + tid] : 0.f;
      pp = v ? p.qpos[r0 + tid] : kPosMinQ;
    }
  };
  auto put = [&](QBlock<DP>& s) {
    T::put(s.q, tid, pq);
    T::put(s.g, tid, pg);
    if (tid < kRows) {
      s.lse2[tid] = (pl == -INFINITY) ? 0.f : pl * kLog2e;
      s.del[tid] = pd;
      s.qp[tid] = pp;
    }
  };

  // S and dP of one block, and the bf16 words of P and dS of two blocks (set = block parity; [t][w]
  // holds registers 8t + 2w, 8t + 2w + 1)
  f32x16 sc, dpc;
  uint32_t pw[2][2][4], dw[2][2][4];

  // One phase (block i in ring slot u). Its first 4 NB slots each issue one dV/dK product of block
  // i - 1 (query half t = k / (2 NB), column block (k mod 2 NB) / 2, dV for even k) while the vector
  // units turn S(i) and dP(i) into the bf16 words of set C; its last 2 NS slots issue S and dP of
  // block i + 1 (k-step k / 2, S for even k) into the same registers, whose old values are then dead.
  auto phase = [&](auto c_c, auto m_c, auto u_c) {
    constexpr int C = decltype(c_c)::value, N = C ^ 1;
    constexpr bool MASKED = decltype(m_c)::value;
    constexpr int NA = 4 * NB;  // slots with vector work
    constexpr int u = decltype(u_c)::value;  // ring slot of block i: a constant, so that operand
                                             // addresses fold the slot into the instruction offset
    const QBlock<DP>& cur = ring[u];
    const QBlock<DP>& prv = ring[(u + kRing - 1) % kRing];
    const QBlock<DP>& nxt = ring[(u + 1) % kRing];
    // tables of block i: registers 4j .. 4j+3 hold queries 8j + 4h .. +3; group j is read kRA slots
    // before the slot that first uses it
    f32x4 ls[4], de[4];
    i32x4 qq[4];
    auto read_tables = [&](int jj) {
      ls[jj] = *(const f32x4*)(cur.lse2 + 8 * jj + 4 * h);
      de[jj] = *(const f32x4*)(cur.del + 8 * jj + 4 * h);
      if (MASKED) qq[jj] = *(const i32x4*)(cur.qp + 8 * jj + 4 * h);
    };
    bf16x8 opa[NMF];
    auto read_op = [&](int sl) {
      if (sl < NA) {
        opa[sl] = T::cols_frag((sl & 1) ? prv.q : prv.g, LL, (sl % (2 * NB)) >> 1, sl / (2 * NB));
      } else {
        const int k = sl - NA;
        opa[sl] = T::rows_frag((k & 1) ? nxt.g : nxt.q, LL, k >> 1);
      }
    };
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (vec_slot(4 * jj, NA) - kRA <= 0) read_tables(jj);
#pragma unroll
    for (int sl = 0; sl < kRA; ++sl) read_op(sl);
    float xp[16], xd[16];
#pragma unroll
    for (int sl = 0; sl < NMF; ++sl) {
      if (sl + kRA < NMF) read_op(sl + kRA);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (vec_slot(4 * jj, NA) - kRA == sl && sl > 0) read_tables(jj);
      if (sl < NA) {
        const int t = sl / (2 * NB), db = (sl % (2 * NB)) >> 1;
        if (sl & 1)
          dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], words_bf16x8(dw[N][t]), dkT[db], 0, 0, 0);
        else
          dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], words_bf16x8(pw[N][t]), dvT[db], 0, 0, 0);
      } else {
        const int k = sl - NA, st = k >> 1;
        if (k & 1)
          dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], vf[st], st == 0 ? f32x16{} : dpc, 0, 0, 0);
        else
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], kf[st], st == 0 ? f32x16{} : sc, 0, 0, 0);
      }
      // Vector work on registers [16 s / NA, 16 (s + 1) / NA) of S(i) and dP(i), in two stages so that
      // a slot's instructions do not wait on each other: P in slot s, then dS and the bf16 words of each
      // finished pair in slot s + 1 (the last of these runs in the first S/dP slot, before dP is
      // overwritten one slot later).
      if (sl >= 1 && sl - 1 < NA) {
#pragma unroll
        for (int r = 16 * (sl - 1) / NA; r < 16 * sl / NA; ++r) {
          xd[r] = xp[r] * (dpc[r] - de[r >> 2][r & 3]);
          if (r & 1) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 a2 = {(__bf16)xp[r - 1], (__bf16)xp[r]};
            const bf16x2 d2 = {(__bf16)xd[r - 1], (__bf16)xd[r]};
            uint32_t& wa = pw[C][r >> 3][(r & 7) >> 1];
            uint32_t& wd = dw[C][r >> 3][(r & 7) >> 1];
            wa = __builtin_bit_cast(uint32_t, a2);
            wd = __builtin_bit_cast(uint32_t, d2);
            asm volatile("" : "+v"(wa), "+v"(wd));
          }
        }
      }
      if (sl < NA) {
#pragma unroll
        for (int r = 16 * sl / NA; r < 16 * (sl + 1) / NA; ++r) {
          const int jj = r >> 2, e = r & 3;
          xp[r] = __builtin_amdgcn_exp2f(sc[r] * p.c2 - ls[jj][e]);
          if (MASKED) xp[r] = (kp <= qq[jj][e]) ? xp[r] : 0.f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A slot that receives no block (the walk has ended) gets lse = +inf and positions that see no key, so
  // a phase over it makes zero P and dS with or without the mask; its Q and dO hold zeros or an older
  // block's rows, always finite.
  auto put_none = [&](QBlock<DP>& s) {
    if (tid < kRows) {
      s.lse2[tid] = INFINITY;
      s.del[tid] = 0.f;
      s.qp[tid] = kPosMinQ;
    }
  };

  // Phases run four at a time until one whose block does not exist: phase n adds dV/dK of the last
  // block n - 1, and phases past it add zeros. MASKED: compare positions for every score.
  auto walk = [&](auto m_c) {
  int cg = 0, cqb = -1;
  if (advance(cg, cqb)) {
    {
      u32x4* z = (u32x4*)ring;
      constexpr int N16 = (int)(sizeof(ring) / 16);
      for (int k = tid; k < N16; k += kBwdThreads) z[k] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    fetch(cg, cqb);
    put(ring[0]);
    bool ok0 = true, ok1 = advance(cg, cqb), ok2 = false;
    if (ok1) {
      fetch(cg, cqb);
      put(ring[1]);
      ok2 = advance(cg, cqb);
    } else {
      put_none(ring[1]);
    }
    if (ok2) fetch(cg, cqb);  // written to its slot by the first iteration
    __syncthreads();
    sc = f32x16{};
    dpc = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::rows_frag(ring[0].q, LL, st), kf[st], sc, 0, 0, 0);
      dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::rows_frag(ring[0].g, LL, st), vf[st], dpc, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[1][t][w] = dw[1][t][w] = 0u;

    auto step = [&](auto c_c, auto u_c) {  // u_c: ring slot of block i
      constexpr int u = decltype(u_c)::value;
      if (ok2)
        put(ring[(u + 2) % kRing]);
      else
        put_none(ring[(u + 2) % kRing]);
      bool ok3 = false;
      if (ok2 && advance(cg, cqb)) {
        ok3 = true;
        fetch(cg, cqb);  // in flight during the phase
      }
      phase(c_c, m_c, u_c);
      __syncthreads();
      const bool real = ok0;
      ok0 = ok1;
      ok1 = ok2;
      ok2 = ok3;
      return real;
    };
    // four steps per iteration (one per ring slot), leaving the loop only after the fourth: a walk
    // ends with up to four phases over blocks that do not exist, which add zeros
    bool more;
    do {
      step(BIntC<0>{}, BIntC<0>{});
      step(BIntC<1>{}, BIntC<1>{});
      step(BIntC<0>{}, BIntC<2>{});
      more = step(BIntC<1>{}, BIntC<3>{});
    } while (more);
  }
  };
  // A workgroup none of whose query blocks straddles its keys (every visited block sees all of them)
  // walks without the mask; the test is one pass over the block bounds, shared by the threads.
  bool need_mask = false;
  if constexpr (CAUSAL) {
    for (int qb = tid; qb < n_qb; qb += kBwdThreads)
      need_mask = need_mask || (p.qblk[2 * qb + 1] >= kmin && p.qblk[2 * qb] < kmax);
    need_mask = __syncthreads_or(need_mask);
  }
  if (need_mask)
    walk(std::true_type{});
  else
    walk(std::false_type{});

  // lane writes its key's row: block db, registers 4i .. 4i+3 are columns db*32 + 8i + 4h .. +3
  if (kvalid) {
    float* dkr = p.dk + (((int64_t)b * p.Hkv + hk) * p.Lk + j) * p.d;
    float* dvr = p.dv + (((int64_t)b * p.Hkv + hk) * p.Lk + j) * p.d;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = db * 32 + 8 * i + 4 * h;
        if (col < p.d) {
          const f32x4 kv = {dkT[db][4 * i] * p.scale, dkT[db][4 * i + 1] * p.scale, dkT[db][4 * i + 2] * p.scale,
                            dkT[db][4 * i + 3] * p.scale};
          const f32x4 vv = {dvT[db][4 * i], dvT[db][4 * i + 1], dvT[db][4 * i + 2], dvT[db][4 * i + 3]};
          *(f32x4*)(dkr + col) = kv;
          *(f32x4*)(dvr + col) = vv;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dQ of 128 query rows per workgroup, software-pipelined over key tiles in the
// same way as dK/dV: key tiles pass through a ring of four LDS slots (K, V and
// key positions of 32 keys); phase i issues the dQ products of tile i - 1
// while the vector units turn S(i), dP(i) into the bf16 dS of set i mod 2, then
// S/dP of tile i + 1; one barrier per tile. With the causal mask every score
// is masked by position (keys past the end and tiles past the walk have
// position "after everything"). Without it no score is masked: the exponent
// is clamped at 0 (lse is at least every score, so this only absorbs
// rounding), which keeps exp(-lse) of a missing key, whose K and V rows are
// zero, finite, and tiles past the walk get zero K rows, so their products
// add nothing.

template <int DP>
struct KTile {
  __bf16 k[kRows * Tile<DP>::RS];
  __bf16 v[kRows * Tile<DP>::RS];
  int kp[kRows];
};

template <int DP, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void dq_kernel(BwdParams p) {
  using T = Tile<DP>;
  constexpr int NS = DP / 16;
  constexpr int NB = DP / 32;
  constexpr int PER = T::PER;
  constexpr int NA = 2 * NB;            // dQ products per phase (slots with vector work)
  constexpr int NMF = NA + 2 * NS;      // MFMAs per phase
  constexpr int kRA = 2;                // slots between an operand read and its MFMA
  __shared__ __attribute__((aligned(16))) KTile<DP> ring[kRing];
  __shared__ int qmax_red[2 * kBwdWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const typename T::Lanes LL = T::lanes(lane);
  const int n_qt = (int)((p.Lq + kGroupRows - 1) / kGroupRows);
  const int item = CAUSAL ? xcd_item(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  // causal: later queries see more keys, so their tiles start first
  const int qt = CAUSAL ? n_qt - 1 - item % n_qt : item % n_qt;
  const int rest = item / n_qt;
  const int bh = rest % (p.B * p.Hq), split = rest / (p.B * p.Hq);
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int hk = hq / (p.Hq / p.Hkv);

  // this lane's query: Q and dO rows as B operands, lse, delta and position
  const int64_t i = (int64_t)qt * kGroupRows + wave * kRows + (lane & 31);
  const bool qvalid = i < p.Lq;
  const int64_t row = ((int64_t)b * p.Hq + hq) * p.Lq + (qvalid ? i : 0);
  bf16x8 qf[NS], gf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int col = 16 * s + 8 * h;
    u32x4 qraw = {0u, 0u, 0u, 0u}, graw = {0u, 0u, 0u, 0u};
    if (qvalid && col < p.d) {
      qraw = *(const u32x4*)(p.q + row * p.d + col);
      graw = *(const u32x4*)(p.dout + row * p.d + col);
    }
    qf[s] = __builtin_bit_cast(bf16x8, qraw);
    gf[s] = __builtin_bit_cast(bf16x8, graw);
  }
  const float lsev = qvalid ? p.lse[row] : 0.f;
  const float lse2 = (lsev == -INFINITY) ? 0.f : lsev * kLog2e;
  const float del = qvalid ? p.delta[row] : 0.f;
  const int qp = qvalid ? p.qpos[i] : kPosMinQ;
  int wq = qp;
  for (int o = 32; o > 0; o >>= 1) wq = max(wq, __shfl_xor(wq, o));
  if (lane == 0) qmax_red[wave] = wq;
  __syncthreads();
  int qmax = qmax_red[0];
  for (int w = 1; w < kBwdWaves; ++w) qmax = max(qmax, qmax_red[w]);

  f32x16 dqT[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) dqT[db] = f32x16{};

  // key tiles of 32 in list order (this workgroup's range of them when the key range is split),
  // skipping tiles after every query of the workgroup; never called again once it has returned false
  const int n_kt_all = (int)((p.Lk + kRows - 1) / kRows);
  const int per_split = (n_kt_all + p.dq_split - 1) / p.dq_split;
  const int t_beg = split * per_split;
  const int n_kt = min(n_kt_all, t_beg + per_split);
  auto advance = [&](int& t) {
    while (++t < n_kt)
      if (!CAUSAL || cload(p.ktile + 2 * t) <= qmax) return true;
    return false;
  };
  // The chunk that holds a tile's first key is tracked by a cursor that is the same for every lane
  // (its descriptor reads are scalar and cached); a tile inside that chunk takes its row addresses
  // from it directly, and only a tile that crosses a chunk end looks up each row's chunk (per-piece
  // cursors that only move forward).
  int cc = 0;
  int cur[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) cur[k] = 0;
  u32x4 pk[PER], pv[PER];
  int pkp = kPosMax;
  auto fetch = [&](int t) {
    const int64_t j0 = (int64_t)t * kRows;
    const cchunk_ptr chunks = (cchunk_ptr)p.chunks;
    while (cc + 1 < p.n_chunks && j0 >= chunks[cc].start + chunks[cc].len) ++cc;
    const BwdChunk ch = chunk_at(p.chunks, cc);
    // the whole tile in one chunk whose 32 rows span less than 2 GB: a base address shared by all
    // lanes plus 32-bit lane offsets
    const bool inside = j0 + kRows <= ch.start + ch.len && ch.ss <= (0x7fffffff / (2 * kRows));
    const int64_t tile_off = (int64_t)b * ch.sb + (int64_t)hk * ch.sh + (j0 - ch.start) * ch.ss;
    const char* kbase = (const char*)((const __bf16*)ch.k + tile_off);
    const char* vbase = (const char*)((const __bf16*)ch.v + tile_off);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int r, c8;
      pk[k] = u32x4{0u, 0u, 0u, 0u};
      pv[k] = u32x4{0u, 0u, 0u, 0u};
      if (T::piece(tid, k, r, c8) && j0 + r < p.Lk && c8 * 8 < p.d) {
        if (inside) {
          const uint32_t off = (uint32_t)r * (uint32_t)(2 * ch.ss) + (uint32_t)(c8 * 16);
          pk[k] = *(const u32x4*)(kbase + off);
          pv[k] = *(const u32x4*)(vbase + off);
        } else {
          cur[k] = max(cur[k], cc);
          const int64_t off = key_offset(p, j0 + r, b, hk, cur[k]);
          pk[k] = gload16(chunk_k(p, cur[k]) + off + c8 * 8);
          pv[k] = gload16(chunk_v(p, cur[k]) + off + c8 * 8);
        }
      }
    }
    if (CAUSAL && tid < kRows) pkp = (j0 + tid < p.Lk) ? p.kpos[j0 + tid] : kPosMax;
  };
  auto put = [&](KTile<DP>& s) {
    T::put(s.k, tid, pk);
    T::put(s.v, tid, pv);
    if (CAUSAL && tid < kRows) s.kp[tid] = pkp;
  };
  // a slot that receives no tile: keys after everything (causal), or zero K rows (not causal), so the
  // products of its tile add nothing
  auto put_none = [&](KTile<DP>& s) {
    if constexpr (CAUSAL) {
      if (tid < kRows) s.kp[tid] = kPosMax;
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      u32x4 zr[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) zr[k] = z;
      T::put(s.k, tid, zr);
    }
  };

  // S^T and dP^T of one tile (lane: query lane % 32, registers: keys out_row(r)), and the bf16 words of
  // dS of two tiles (set = tile parity; [t][w] holds registers 8t + 2w, 8t + 2w + 1)
  f32x16 sc, dpc;
  uint32_t dw[2][2][4];

  // One phase (tile i in ring slot u): NA slots of dQ products of tile i - 1 (key half t = k / NB,
  // column block k mod NB) with the vector work on S(i), dP(i), then 2 NS slots of S and dP of tile
  // i + 1 (k-step k / 2, S for even k) into the same registers.
  auto phase = [&](auto c_c, auto u_c) {
    constexpr int C = decltype(c_c)::value, N = C ^ 1;
    constexpr int u = decltype(u_c)::value;  // ring slot of tile i: a constant, as in the dK/dV kernel
    const KTile<DP>& cur_t = ring[u];
    const KTile<DP>& prv = ring[(u + kRing - 1) % kRing];
    const KTile<DP>& nxt = ring[(u + 1) % kRing];
    i32x4 kk[4];  // key positions of registers 4j .. 4j+3: keys 8j + 4h .. +3
    auto read_keys = [&](int jj) {
      if (CAUSAL) kk[jj] = *(const i32x4*)(cur_t.kp + 8 * jj + 4 * h);
    };
    bf16x8 opa[NMF];
    auto read_op = [&](int sl) {
      if (sl < NA) {
        opa[sl] = T::cols_frag(prv.k, LL, sl % NB, sl / NB);
      } else {
        const int k = sl - NA;
        opa[sl] = T::rows_frag((k & 1) ? nxt.v : nxt.k, LL, k >> 1);
      }
    };
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (vec_slot(4 * jj, NA) - kRA <= 0) read_keys(jj);
#pragma unroll
    for (int sl = 0; sl < kRA; ++sl) read_op(sl);
    float xp[16], xd[16];
#pragma unroll
    for (int sl = 0; sl < NMF; ++sl) {
      if (sl + kRA < NMF) read_op(sl + kRA);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (vec_slot(4 * jj, NA) - kRA == sl && sl > 0) read_keys(jj);
      if (sl < NA) {
        const int tt = sl / NB, db = sl % NB;
        dqT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], words_bf16x8(dw[N][tt]), dqT[db], 0, 0, 0);
      } else {
        const int k = sl - NA, st = k >> 1;
        if (k & 1)
          dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], gf[st], st == 0 ? f32x16{} : dpc, 0, 0, 0);
        else
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl], qf[st], st == 0 ? f32x16{} : sc, 0, 0, 0);
      }
      // vector work in two stages as in the dK/dV kernel: P in slot s, dS and its words in slot s + 1
      if (sl >= 1 && sl - 1 < NA) {
#pragma unroll
        for (int r = 16 * (sl - 1) / NA; r < 16 * sl / NA; ++r) {
          xd[r] = xp[r] * (dpc[r] - del);
          if (r & 1) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 d2 = {(__bf16)xd[r - 1], (__bf16)xd[r]};
            uint32_t& wd = dw[C][r >> 3][(r & 7) >> 1];
            wd = __builtin_bit_cast(uint32_t, d2);
            asm volatile("" : "+v"(wd));
          }
        }
      }
      if (sl < NA) {
#pragma unroll
        for (int r = 16 * sl / NA; r < 16 * (sl + 1) / NA; ++r)
          if (CAUSAL)
            xp[r] = (kk[r >> 2][r & 3] <= qp) ? __builtin_amdgcn_exp2f(sc[r] * p.c2 - lse2) : 0.f;
          else
            xp[r] = __builtin_amdgcn_exp2f(fminf(sc[r] * p.c2 - lse2, 0.f));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phases run four at a time until one whose tile does not exist: phase n adds dQ of the last tile
  // n - 1, and phases past it add zeros.
  int t = t_beg - 1;
  if (advance(t)) {
    {
      u32x4* z = (u32x4*)ring;
      constexpr int N16 = (int)(sizeof(ring) / 16);
      for (int k = tid; k < N16; k += kBwdThreads) z[k] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    fetch(t);
    put(ring[0]);
    bool ok0 = true, ok1 = advance(t), ok2 = false;
    if (ok1) {
      fetch(t);
      put(ring[1]);
      ok2 = advance(t);
    } else {
      put_none(ring[1]);
    }
    if (ok2) fetch(t);  // written to its slot by the first iteration
    __syncthreads();
    sc = f32x16{};
    dpc = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::rows_frag(ring[0].k, LL, st), qf[st], sc, 0, 0, 0);
      dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::rows_frag(ring[0].v, LL, st), gf[st], dpc, 0, 0, 0);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int w = 0; w < 4; ++w) dw[1][tt][w] = 0u;

    auto step = [&](auto c_c, auto u_c) {  // u_c: ring slot of tile i
      constexpr int u = decltype(u_c)::value;
      if (ok2)
        put(ring[(u + 2) % kRing]);
      else
        put_none(ring[(u + 2) % kRing]);
      bool ok3 = false;
      if (ok2 && advance(t)) {
        ok3 = true;
        fetch(t);  // in flight during the phase
      }
      phase(c_c, u_c);
      __syncthreads();
      const bool real = ok0;
      ok0 = ok1;
      ok1 = ok2;
      ok2 = ok3;
      return real;
    };
    // four steps per iteration, one per ring slot (up to four trailing phases add zeros)
    bool more;
    do {
      step(BIntC<0>{}, BIntC<0>{});
      step(BIntC<1>{}, BIntC<1>{});
      step(BIntC<0>{}, BIntC<2>{});
      more = step(BIntC<1>{}, BIntC<3>{});
    } while (more);
  }

  if (qvalid) {
    // one range: dQ itself; several: this range's unscaled partial, summed by dq_reduce_kernel
    const bool direct = p.dq_split == 1;
    const float sc_out = direct ? p.scale : 1.f;
    float* dqr = direct ? p.dq + row * p.d
                        : p.dq_part + ((int64_t)split * p.B * p.Hq * p.Lq + row) * p.d;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int col = db * 32 + 8 * k + 4 * h;
        if (col < p.d) {
          const f32x4 v = {dqT[db][4 * k] * sc_out, dqT[db][4 * k + 1] * sc_out, dqT[db][4 * k + 2] * sc_out,
                           dqT[db][4 * k + 3] * sc_out};
          *(f32x4*)(dqr + col) = v;
        }
      }
  }
}

// dQ = scale * (sum of the key-range partials, in range order); 16 bytes per thread.
__global__ __launch_bounds__(256) void dq_reduce_kernel(int64_t n4, int ns, const f32x4* __restrict__ part,
                                                        f32x4* __restrict__ dq, float scale) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n4) return;
  f32x4 acc = part[e];
  for (int s = 1; s < ns; ++s) acc += part[(int64_t)s * n4 + e];
  dq[e] = acc * scale;
}

// ---------------------------------------------------------------------------
// Position tables of a call, built on the device from the chunk and query
// segment descriptors: the global position of every query row and key (or the
// "sees everything" values without a causal mask), and the smallest and largest
// position of every 32-row query block and 32-key tile. Thread t < nqb builds
// query block t, thread nqb + u builds key tile u.

struct BwdSeg {
  int64_t row0, len, pos0, ps;
};
static_assert(sizeof(BwdChunk) % 4 == 0 && sizeof(BwdSeg) % 4 == 0, "tables are uploaded in 4-byte words");

__global__ __launch_bounds__(256) void bwd_positions_kernel(const BwdChunk* __restrict__ chunks, int n_chunks,
                                                            const BwdSeg* __restrict__ segs, int n_segs,
                                                            int64_t lq, int64_t lk, int causal, int* __restrict__ qpos,
                                                            int* __restrict__ kpos, int* __restrict__ qblk,
                                                            int* __restrict__ ktile) {
  const int64_t nqb = (lq + kRows - 1) / kRows, nkt = (lk + kRows - 1) / kRows;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < nqb) {
    const int64_t i0 = t * kRows, i1 = min(lq, i0 + kRows);
    int s = 0;
    while (s + 1 < n_segs && i0 >= segs[s].row0 + segs[s].len) ++s;
    int mn = kPosMax, mx = kPosMinQ;
    for (int64_t i = i0; i < i1; ++i) {
      while (s + 1 < n_segs && i >= segs[s].row0 + segs[s].len) ++s;
      const int pos = causal ? (int)(segs[s].pos0 + segs[s].ps * (i - segs[s].row0)) : kPosAllQ;
      qpos[i] = pos;
      mn = min(mn, pos);
      mx = max(mx, pos);
    }
    qblk[2 * t] = mn;
    qblk[2 * t + 1] = mx;
  } else if (t < nqb + nkt) {
    const int64_t u = t - nqb;
    const int64_t j0 = u * kRows, j1 = min(lk, j0 + kRows);
    // last chunk starting at or before key j0 (chunks are non-empty and in list order)
    int lo = 0, hi = n_chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (chunks[mid].start <= j0) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    int mn = kPosMax, mx = kPosMinQ;
    for (int64_t j = j0; j < j1; ++j) {
      while (c + 1 < n_chunks && j >= chunks[c].start + chunks[c].len) ++c;
      const int pos = causal ? (int)(chunks[c].pos0 + (int64_t)chunks[c].ps * (j - chunks[c].start)) : 0;
      kpos[j] = pos;
      mn = min(mn, pos);
      mx = max(mx, pos);
    }
    ktile[2 * u] = mn;
    ktile[2 * u + 1] = mx;
  }
}

// ---------------------------------------------------------------------------
// Host side.

using namespace ra_host;

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t chunks, segs, qpos, kpos, qblk, ktile, table_end, delta, part, total;
  int dq_split;
};

// Key-range split of the dQ kernel: enough workgroups for two per CU, each range
// at least 16 key tiles of 32, at most 8 ranges.
int choose_dq_split(int batch, int q_heads, int64_t q_len, int64_t total_keys) {
  const int64_t base = ((q_len + kGroupRows - 1) / kGroupRows) * (int64_t)batch * q_heads;
  const int64_t tiles = (total_keys + kRows - 1) / kRows;
  int ns = 1;
  while (base > 0 && base * ns < 2 * 256 && ns < 8 && tiles / (2 * ns) >= 16) ns *= 2;
  return ns;
}

BwdLayout bwd_layout(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys, int n_chunks,
                     int n_q_segments) {
  BwdLayout L;
  const int64_t nqb = (q_len + kRows - 1) / kRows, nkt = (total_keys + kRows - 1) / kRows;
  L.chunks = 0;
  L.segs = L.chunks + al256(sizeof(BwdChunk) * (size_t)(n_chunks > 0 ? n_chunks : 1));
  L.qpos = L.segs + al256(sizeof(BwdSeg) * (size_t)(n_q_segments > 0 ? n_q_segments : 1));
  L.kpos = L.qpos + al256(sizeof(int) * (size_t)(q_len > 0 ? q_len : 1));
  L.qblk = L.kpos + al256(sizeof(int) * (size_t)(total_keys > 0 ? total_keys : 1));
  L.ktile = L.qblk + al256(2 * sizeof(int) * (size_t)(nqb > 0 ? nqb : 1));
  L.table_end = L.ktile + al256(2 * sizeof(int) * (size_t)(nkt > 0 ? nkt : 1));
  L.delta = L.table_end;
  const size_t rows = (size_t)(batch > 0 ? batch : 0) * (size_t)(q_heads > 0 ? q_heads : 0) *
                      (size_t)(q_len > 0 ? q_len : 0);
  L.part = L.delta + al256(sizeof(float) * rows);
  L.dq_split = (batch > 0 && q_heads > 0 && q_len > 0) ? choose_dq_split(batch, q_heads, q_len, total_keys) : 1;
  L.total = L.part + (L.dq_split > 1 ? al256(sizeof(float) * (size_t)L.dq_split * rows *
                                             (size_t)(head_dim > 0 ? head_dim : 0))
                                     : 0);
  return L;
}

template <int DP>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t n_kt = (p.Lk + kGroupRows - 1) / kGroupRows;
  const int64_t n_qt = (p.Lq + kGroupRows - 1) / kGroupRows;
  timer_begin(s);
  if (n_kt > 0) {
    const dim3 grid((unsigned)(n_kt * p.B * p.Hkv));
    if (p.causal)
      hipLaunchKernelGGL((dkdv_kernel<DP, true>), grid, dim3(kBwdThreads), 0, s, p);
    else
      hipLaunchKernelGGL((dkdv_kernel<DP, false>), grid, dim3(kBwdThreads), 0, s, p);
  }
  timer_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timer_begin(s);
  {
    const dim3 grid((unsigned)(n_qt * p.B * p.Hq * p.dq_split));
    if (p.causal)
      hipLaunchKernelGGL((dq_kernel<DP, true>), grid, dim3(kBwdThreads), 0, s, p);
    else
      hipLaunchKernelGGL((dq_kernel<DP, false>), grid, dim3(kBwdThreads), 0, s, p);
  }
  timer_end(s);
  e = hipGetLastError();
  if (e != hipSuccess || p.dq_split == 1) return e;
  const int64_t n4 = (int64_t)p.B * p.Hq * p.Lq * p.d / 4;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, n4, p.dq_split,
                     (const f32x4*)p.dq_part, (f32x4*)p.dq, p.scale);
  return hipGetLastError();
}

}  // namespace

extern "C" {

size_t ra_ring_backward_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                                        int n_chunks, int n_q_segments) {
  if (n_chunks < 0) n_chunks = 0;
  if (n_q_segments < 0) n_q_segments = 0;
  if (q_len < 0) q_len = 0;
  if (total_keys < 0) total_keys = 0;
  return bwd_layout(batch, q_heads, head_dim, q_len, total_keys, n_chunks, n_q_segments).total;
}

int ra_ring_attention_backward(int dtype, int batch, int q_heads, int kv_heads, int head_dim, const void* q,
                               const ra_q_segment* q_segments, int n_q_segments, const ra_kv_chunk* chunks,
                               int n_chunks, int causal, float scale, const float* out, const float* lse,
                               const void* dout, void* workspace, size_t workspace_bytes, float* dq, float* dk,
                               float* dv, void* stream) {
  g_err[0] = 0;
  int st = check_dims(dtype, batch, q_heads, kv_heads, head_dim);
  if (st) return st;
  if (dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs");
  if (head_dim % 8 != 0)
    return fail(RA_ERR_UNSUPPORTED, "the backward pass takes head_dim a multiple of 8 (got %d)", head_dim);
  if (n_q_segments < 1 || !q_segments) return fail(RA_ERR_NULL, "at least one query segment is required");
  if (n_chunks < 0 || (n_chunks > 0 && !chunks)) return fail(RA_ERR_NULL, "chunk array missing");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RA_ERR_SHAPE, "scale must be finite and > 0");
  int64_t lq = 0;
  for (int s = 0; s < n_q_segments; ++s) {
    const ra_q_segment& g = q_segments[s];
    if (g.len < 0) return fail(RA_ERR_SHAPE, "query segment %d: negative length", s);
    if (g.pos_stride < 0) return fail(RA_ERR_SHAPE, "query segment %d: negative pos_stride", s);
    if (causal && g.len > 0 && !positions_fit(g.global_offset, g.len, pos_step(g.pos_stride)))
      return fail(RA_ERR_SHAPE, "query segment %d: positions outside [0, 2^31-1)", s);
    lq += g.len;
  }
  int64_t lk = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if ((st = check_chunk(chunks[c], c, head_dim))) return st;
    if (chunks[c].len > 0 && !chunk_vec_ok(chunks[c], head_dim, 2))
      return fail(RA_ERR_UNSUPPORTED, "chunk %d: rows must be 16-byte aligned for the backward pass", c);
    lk += chunks[c].len;
  }
  if (lk > kPosLimit) return fail(RA_ERR_UNSUPPORTED, "more than 2^31-2 keys in total");
  if (lq == 0 || batch == 0) return RA_OK;
  if (!q || !out || !lse || !dout || !dq) return fail(RA_ERR_NULL, "q, out, lse, dout and dq must be non-null");
  if (lk > 0 && (!dk || !dv)) return fail(RA_ERR_NULL, "dk and dv must be non-null");
  if (!vec_ok(q, head_dim, head_dim, 2) || !vec_ok(dout, head_dim, head_dim, 2) || (uintptr_t)out % 16 != 0 ||
      (uintptr_t)dq % 16 != 0 || (lk > 0 && ((uintptr_t)dk % 16 != 0 || (uintptr_t)dv % 16 != 0)))
    return fail(RA_ERR_UNSUPPORTED, "q, dout, out, dq, dk and dv must be 16-byte aligned");
  const int64_t blocks_q = ((lq + kGroupRows - 1) / kGroupRows) * batch * q_heads;
  const int64_t blocks_k = ((lk + kGroupRows - 1) / kGroupRows) * batch * kv_heads;
  if (blocks_q > 0x7fffffffLL || blocks_k > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "grid too large");
  const BwdLayout L = bwd_layout(batch, q_heads, head_dim, lq, lk, n_chunks, n_q_segments);
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % 256 != 0)
    return fail(RA_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total,
                workspace_bytes);

  // Chunk and query-segment descriptors go to the workspace as kernel arguments
  // (host arrays are read only during this call); the position tables are then
  // built from them on the device.
  hipStream_t hs = (hipStream_t)stream;
  TableUpload up(workspace, hs);
  int nc = 0;
  int64_t start = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const ra_kv_chunk& ch = chunks[c];
    if (ch.len == 0) continue;
    BwdChunk d = {};
    d.k = ch.k;
    d.v = ch.v;
    d.start = start;
    d.len = ch.len;
    d.sb = ch.stride_b;
    d.sh = ch.stride_h;
    d.ss = ch.stride_s;
    d.pos0 = (int32_t)ch.global_offset;
    d.ps = (int32_t)pos_step(ch.pos_stride);
    up.put(&d, sizeof(d));
    ++nc;
    start += ch.len;
  }
  up.zero_to(L.segs);
  int64_t row0 = 0;
  for (int s = 0; s < n_q_segments; ++s) {
    BwdSeg g = {};
    g.row0 = row0;
    g.len = q_segments[s].len;
    g.pos0 = q_segments[s].global_offset;
    g.ps = pos_step(q_segments[s].pos_stride);
    up.put(&g, sizeof(g));
    row0 += q_segments[s].len;
  }
  up.zero_to(L.qpos);
  hipError_t e = up.finish();
  if (e != hipSuccess) return hip_fail(e, "ring_attention_backward descriptor upload");
  {
    char* ws = (char*)workspace;
    const int64_t nthreads = (lq + kRows - 1) / kRows + (lk + kRows - 1) / kRows;
    hipLaunchKernelGGL(bwd_positions_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, hs,
                       (const BwdChunk*)(ws + L.chunks), nc, (const BwdSeg*)(ws + L.segs), n_q_segments, lq, lk,
                       causal ? 1 : 0, (int*)(ws + L.qpos), (int*)(ws + L.kpos), (int*)(ws + L.qblk),
                       (int*)(ws + L.ktile));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "ring_attention_backward position tables launch");
  }

  BwdParams p = {};
  char* ws = (char*)workspace;
  p.q = (const __bf16*)q;
  p.dout = (const __bf16*)dout;
  p.out = out;
  p.lse = lse;
  p.delta = (float*)(ws + L.delta);
  p.qpos = (const int*)(ws + L.qpos);
  p.kpos = (const int*)(ws + L.kpos);
  p.qblk = (const int*)(ws + L.qblk);
  p.ktile = (const int*)(ws + L.ktile);
  p.chunks = (const BwdChunk*)(ws + L.chunks);
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.Lq = lq;
  p.Lk = lk;
  p.n_chunks = nc > 0 ? nc : 1;
  p.B = batch;
  p.Hq = q_heads;
  p.Hkv = kv_heads;
  p.d = head_dim;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.c2 = scale * kLog2e;
  p.dq_split = L.dq_split;
  p.dq_part = L.dq_split > 1 ? (float*)(ws + L.part) : nullptr;

  const int64_t rows = (int64_t)batch * q_heads * lq;
  int lpr = 1, sh = 0;
  while (lpr < head_dim / 8) {
    lpr <<= 1;
    ++sh;
  }
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)((rows * lpr + 255) / 256)), dim3(256), 0, hs, rows, head_dim,
                     lpr, sh, (const __bf16*)dout, out, p.delta);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "ring_attention_backward delta launch");
  // tiles are DP = 32, 64 or 128 columns wide; columns past head_dim are zero in LDS and registers
  // and are never written out
  if (head_dim <= 32)
    e = launch_bwd<32>(p, hs);
  else if (head_dim <= 64)
    e = launch_bwd<64>(p, hs);
  else
    e = launch_bwd<128>(p, hs);
  if (e != hipSuccess) return hip_fail(e, "ring_attention_backward launch");
  return RA_OK;
}

}  // extern "C"
