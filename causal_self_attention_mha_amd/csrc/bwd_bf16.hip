// bf16 causal attention backward on gfx950 MFMA: a split pass with no atomics.
//
// For the loss L with dL/do = dout (and no gradient through lse), per (b, h):
//   delta_i = <dout_i, o_i>
//   P_ij = exp(s <q_i, k_j> - lse_i) for j <= i, else 0
//   dP_ij = <dout_i, v_j>,   dS_ij = P_ij (dP_ij - delta_i)
//   dv_j = sum_i P_ij dout_i,  dk_j = s sum_i dS_ij q_i,  dq_i = s sum_j dS_ij k_j
// i.e. the gradient of the flash_attn_func(q, k, v, causal=True) call that
// nanochat trains through (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法",
// section 5 "Flash Attention integration").
//
// Three kernels on one stream:
//   delta_kernel    rowsum(dout * o)                      (HBM bound)
//   dkdv_kernel     a 128-key tile per work item; K and V stay in registers
//                   as MFMA operands, query tiles of 64 are copied HBM -> LDS
//                   (triple-buffered, read row-wise and transposed);
//                   accumulates dK, dV and, given a workspace, stores dS
//   dq_gemm_kernel  with the dS workspace: a 256-query tile per work item,
//                   dQ = s dS K over the stored blocks
// Both run persistent workgroups (one per compute unit) that walk their
// work items in a balanced order (persistent_item).
//   dq_kernel       without it: one workgroup per 128-query tile; Q, dout stay
//                   in registers, key tiles of 64 stream through LDS, S and dP
//                   are recomputed; accumulates dQ
// P and dS are rounded to bf16 before they enter an MFMA; everything else is
// fp32.  Each output element is written by exactly one lane, so results are
// bitwise deterministic.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

// o and dout are read once by the delta kernel and dk, dv written once by
// the dK/dV pass: non-temporal policy for both (bit 1: delta's loads,
// 66.9 -> 55.5 us at d20; bit 4: the dK/dV stores, which leaves the caches
// to the dQ GEMM's K and dS: dq 341.6 -> 332.3 us).  Bit 8 (the dK/dV
// pass's copies of an item's K and V rows, also read once) measured no gain
// (dq 331 -> 335 us) and is off.  The forward's O stores (8 bytes per lane)
// became much slower with it (410 -> 582 us) and keep the default policy.
#ifndef NA_NT_EXTRA
#define NA_NT_EXTRA 5
#endif

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- delta

// 16 lanes per row, 16 rows per 256-thread workgroup.  Rows are walked in
// (b, h, t) order, t fastest, so the fp32 delta stores of neighbouring groups
// are contiguous; each group still reads 256 contiguous bytes of o and dout.
__global__ __launch_bounds__(256) void delta_kernel(const u16* __restrict__ o,
                                                    const u16* __restrict__ dout,
                                                    float* __restrict__ delta, int B, int T,
                                                    int H) {
  const long row = static_cast<long>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const long n_rows = static_cast<long>(B) * T * H;
  if (row >= n_rows) return;  // whole 16-lane groups drop out together
  const int chunk = threadIdx.x & 15;
  const int t = static_cast<int>(row % T);
  const long bh = row / T;
  const int h = static_cast<int>(bh % H);
  const int b = static_cast<int>(bh / H);
  const size_t off = ((static_cast<size_t>(b) * T + t) * H + h) * D + 8 * chunk;
#if NA_NT_EXTRA & 1
  const uint4 a = ld16_nt(o + off);
  const uint4 g = ld16_nt(dout + off);
#else
  const uint4 a = ld16(o + off);
  const uint4 g = ld16(dout + off);
#endif
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = (&a.x)[w], y = (&g.x)[w];
    acc = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
    acc = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), acc);
  }
  acc = sum16(acc);
  if (chunk == 0) delta[row] = acc;  // row == (b * H + h) * T + t
}

// ---------------------------------------------------------------- prologue backward

// With the QK-norm + rotary prologue folded into the backward, the kernels that
// write dq and dk turn the gradient g of a rotated row into the gradient of
// the raw row x (readings of the prologue: z = x r, r = 1 / sqrt(mean(x^2) +
// eps), y = R z with pairs (i, i + 64) turned by +theta):
//   dz = R^T g,  dx = r (dz - z mean(dz z)).
struct RopeBwd {
  const u16* raw;  // the raw q or k, same layout as the gradient
  const float* cos_t;
  const float* sin_t;  // fp32 (>= T, 64) tables, row = position
  float eps;
};

// The inputs of rope_bwd_chunk that come from memory: the raw chunk and the
// lane's eight cos and sin values, loaded ahead of the gradient they meet.
struct RopeRow {
  uint4 x16;
  float4 c0, c1, s0, s1;
};
__device__ __forceinline__ RopeRow rope_row_load(const u16* raw_chunk, const RopeBwd& ra, int pos,
                                                 int c) {
  const size_t tp = static_cast<size_t>(pos) * (D / 2) + 8 * (c & 7);
  RopeRow r;
  r.x16 = raw_chunk != nullptr ? ld16(raw_chunk) : make_uint4(0, 0, 0, 0);
  r.c0 = *reinterpret_cast<const float4*>(ra.cos_t + tp);
  r.c1 = *reinterpret_cast<const float4*>(ra.cos_t + tp + 4);
  r.s0 = *reinterpret_cast<const float4*>(ra.sin_t + tp);
  r.s1 = *reinterpret_cast<const float4*>(ra.sin_t + tp + 4);
  return r;
}

// 16 lanes per 256-byte row, lane c holding elements 8 c .. 8 c + 7: gradient
// chunk g16 of the rotated row, and the raw chunk with the angles of its
// position (RopeRow); returns the raw row's gradient chunk.  Every lane of
// the 16-lane group takes part.
__device__ __forceinline__ uint4 rope_bwd_chunk(uint4 g16, const RopeRow& rw, float eps, int c) {
  const uint4 x16 = rw.x16;
  float g[8], x[8];
  const uint32_t gw[4] = {g16.x, g16.y, g16.z, g16.w}, xw[4] = {x16.x, x16.y, x16.z, x16.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    g[2 * j] = __uint_as_float(gw[j] << 16);
    g[2 * j + 1] = __uint_as_float(gw[j] & 0xffff0000u);
    x[2 * j] = __uint_as_float(xw[j] << 16);
    x[2 * j + 1] = __uint_as_float(xw[j] & 0xffff0000u);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  const float r = __builtin_amdgcn_rsqf(sum16(ss) * (1.f / D) + eps);
  const float cs[8] = {rw.c0.x, rw.c0.y, rw.c0.z, rw.c0.w, rw.c1.x, rw.c1.y, rw.c1.z, rw.c1.w};
  const float sn[8] = {rw.s0.x, rw.s0.y, rw.s0.z, rw.s0.w, rw.s1.x, rw.s1.y, rw.s1.z, rw.s1.w};
  const float sg = c < 8 ? 1.f : -1.f;  // dz_i = g_i c + g_{i+64} s, dz_{i+64} = g_{i+64} c - g_i s
  float dz[8], dot = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gp = dpp<0x128>(g[e]);  // the partner lane's element (row_ror:8)
    dz[e] = fmaf(g[e], cs[e], sg * sn[e] * gp);
    dot = fmaf(dz[e], x[e], dot);
  }
  const float m = sum16(dot) * r * (1.f / D);  // mean(dz z)
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = r * fmaf(-x[e] * r, m, dz[e]);
  return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                    pack_bf16x2(y[6], y[7]));
}

// With the value-embedding gate's backward folded in as well (v' = v + 3
// sigmoid(g) ve fed the attention as its values), the kernel that writes dv
// (= dv') also writes dve = 3 sigmoid(g) dv' and dg = 3 sigmoid(g)
// (1 - sigmoid(g)) <ve, dv'>, from the bf16 dv' it stores, with the
// arithmetic of the separate value-gate backward.
struct GateBwd {
  const u16* ve;    // (B, T, Hk, D), as v
  const u16* gate;  // (B, T, Hk) logits
  u16* dve;         // as ve
  u16* dgate;       // as gate
};

// ---------------------------------------------------------------- dK, dV

constexpr int KT_KEYS = 128;  // keys per workgroup (32 per wavefront)
constexpr int QT_ROWS = 64;   // queries per LDS tile
constexpr int NBUF = 3;       // query tiles resident in LDS at once
constexpr uint32_t TILE_B = kTileBytes;      // one 64 x 128 bf16 tile
constexpr uint32_t BUF_B = 2 * TILE_B;        // one buffer: q tile, then dout tile

// Query tiles are copied straight from HBM into LDS (no register staging, no
// transposed copy) in the swizzled 64 x 128 layout of tile_swz; Q and dout rows
// are read row-wise as MFMA A operands and transposed as B operands.

// Initial values of one 32-query block's score chains, for this lane's
// accumulator elements (element r: query row row0 + acc_row(lane, r), see
// dkdv_scores): the S chain starts at -lse log2(e) and the dP chain at -delta,
// so that the finished chains hold the exponent of P and dP - delta.  ini is
// the LDS byte address of the wavefront's rewritten rows of the block's tile
// (-lse log2 e at +0, -delta at +256); rows row0 + 8 half + 0..7 and
// row0 + 16 + 8 half + 0..7 are two runs of 32 bytes.
__device__ __forceinline__ void load_chain_init(uint32_t ini, int row0, int lane, f32x16& s,
                                                f32x16& p) {
  const uint32_t a = ini + 4 * (row0 + 8 * (lane >> 5));
  const uint4 s0 = lds_ld16(a), s1 = lds_ld16(a + 16), s2 = lds_ld16(a + 64), s3 = lds_ld16(a + 80);
  const uint4 d0 = lds_ld16(a + 256), d1 = lds_ld16(a + 272), d2 = lds_ld16(a + 320),
              d3 = lds_ld16(a + 336);
  s = __builtin_bit_cast(f32x16, (u32x16{s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w, s2.x,
                                          s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w}));
  p = __builtin_bit_cast(f32x16, (u32x16{d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w, d2.x,
                                          d2.y, d2.z, d2.w, d3.x, d3.y, d3.z, d3.w}));
}

// Link i of a score chain (the first one waits out a VALU write of the
// chain's initial value).
__device__ __forceinline__ void mfma_chain_first_or_next(int i, f32x16& d, bf16x8 a, bf16x8 b) {
  if (i == 0)
    mfma_chain_first(d, a, b);
  else
    mfma_chain(d, a, b);
}

// One 32-query block of a dK/dV step for one wavefront (32 keys), in three
// phases:
//   scores:  S' = Q K'^T - lse log2 e, dP' = dout V^T - delta (A = Q / dout
//            rows from LDS, B = K' / V in AGPRs, K' = s log2(e) K rounded to
//            bf16; the chains start from load_chain_init; lane: key, element
//            r: query acc_row(lane, r))
//   probs:   P = exp2(S'), dS = P dP', rounded to bf16
//   accum:   dV^T += dout^T P, dK^T += Q^T dS  (A = query tiles read
//            transposed, B = P / dS from registers; lane: key, element r: d)
// Every MFMA here takes one 1 KB operand from LDS, so the compute unit's LDS
// read bandwidth (about 4 KB per MFMA time with four wavefronts, close to what
// it delivers) bounds the pass: the reads are spread evenly over the step's 32
// MFMAs, and each is issued several MFMAs before its use (a single wavefront
// per SIMD has no other wavefront to hide LDS latency).
//
// Row operands of a block's score chains: rows row0 + perm rows of the tile
// behind na, 16-element chunks kc; Q at +0, dout at + TILE_B.
__device__ __forceinline__ void read_rows(const uint32_t (&na)[8], int row0, int kc, bf16x8& q,
                                          bf16x8& g) {
  q = as_bf16x8(lds_ld16(na[kc] + row0 * 256));
  g = as_bf16x8(lds_ld16(na[kc] + row0 * 256 + TILE_B));
}

// Scores of one block without a preceding step (the first block of a
// wavefront's diagonal): its chains (init from ini, rows of na at row0) into
// sacc, pacc, and, for the step that follows, the initial values of the next
// block's chains (ini1 at row1) and its first row operands (na1 at row1).
// On return sacc, pacc hold finished chains (16 wait states after the last
// MFMA; see mfma_chain).
__device__ __forceinline__ void dkdv_scores(const uint32_t (&na)[8], int row0, uint32_t ini,
                                            const uint32_t (&na1)[8], int row1, uint32_t ini1,
                                            const bf16x8 (&kreg)[8], const bf16x8 (&vreg)[8],
                                            f32x16& sacc, f32x16& pacc, f32x16& s1, f32x16& p1,
                                            bf16x8 (&pre)[8], int lane) {
  load_chain_init(ini, row0, lane, sacc, pacc);
#pragma unroll
  for (int k4 = 0; k4 < 8; k4 += 4) {
    bf16x8 aq[4], ag[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) read_rows(na, row0, k4 + i, aq[i], ag[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (k4 + i == 0) {
        mfma_chain_first(sacc, aq[i], kreg[k4 + i]);
        mfma_chain_first(pacc, ag[i], vreg[k4 + i]);
      } else {
        mfma_chain(sacc, aq[i], kreg[k4 + i]);
        mfma_chain(pacc, ag[i], vreg[k4 + i]);
      }
    }
  }
  load_chain_init(ini1, row1, lane, s1, p1);
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) read_rows(na1, row1, kc, pre[kc], pre[4 + kc]);
  asm volatile("s_nop 15" : "+v"(sacc), "+v"(pacc));
}

// dS of one 32-query x 32-key block, kept for the dQ GEMM: 1024 bf16, the
// element of key k and query q = 16 j + 8 h + e (e < 8) at 512 j + 16 k + 8 h
// + e, so that a lane's two 16-byte stores (its key, 8 queries each) go to two
// contiguous KiB, one per store instruction.  Stored as a [key][query] matrix,
// each instruction wrote 32-byte pieces 64 bytes apart; the contiguous order
// took the d20 dK/dV pass from 877 to 864 us, and the dQ GEMM, whose copies
// gather each block back into [key][query] order in LDS from two 512-byte
// runs, from 318 to 322 us.  Blocks of a head are packed lower-triangularly:
// block (qblk, kblk), kblk <= qblk, at index qblk (qblk + 1) / 2 + kblk.
__device__ __forceinline__ size_t ds_block_index(int bh, int nbt, int qblk, int kblk) {
  return (static_cast<size_t>(bh) * nbt + qblk * (qblk + 1) / 2 + kblk) * 1024;
}

// The dS blocks are written once and read once, by another kernel: both
// sides use the non-temporal policy (bit 1: the dQ GEMM's copies, bit 2: the
// dK/dV stores), which keeps K and Q tiles, re-read by neighbouring work
// items, in the caches (d20: dq 356.8 -> 338.0 us, dkdv 893 -> 884 us).
#ifndef NA_DS_NT
#define NA_DS_NT 3
#endif
__device__ __forceinline__ void store_ds(u16* blk, const bf16x8 (&sb)[2], int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  // lane: key l32; sb[j]: queries 16 j + 8 half + 0..7
  if constexpr ((NA_DS_NT & 2) != 0) {
    st16_nt(blk + 16 * l32 + 8 * half, __builtin_bit_cast(uint4, sb[0]));
    st16_nt(blk + 512 + 16 * l32 + 8 * half, __builtin_bit_cast(uint4, sb[1]));
  } else {
    st16(blk + 8 * (32 * half + l32), __builtin_bit_cast(uint4, sb[0]));
    st16(blk + 512 + 8 * (32 * half + l32), __builtin_bit_cast(uint4, sb[1]));
  }
}

// Steady-state step: probabilities of the current block (finished chains in
// s_cur, p_cur), score chains of the next block (s_nxt, p_nxt hold their
// initial values and pre[] its first four row operand pairs on entry), then
// the current block's dK/dV accumulation.  The order is fixed by hand,
// separated by scheduling fences: eight rounds, each with one S and one dP
// MFMA, the probability math of two of this lane's sixteen (key, query)
// elements, the row reads of round i + 4 (rounds 0..3) and one transposed
// operand of the accumulation's first chunk; then sixteen accumulation
// MFMAs, during which the second chunk's transposed operands are read (eight
// MFMAs ahead of use) and, for the step after next, the block two ahead's
// initial values (into s_cur, p_cur, dead by then) and first row operands
// (into pre).  The block two ahead sits at the same rows (rowC) of the next
// position's tile: nn, ini_nn.  na/rowN locate the next block, ta/rowC the
// current one.
// MASK: the current block holds this wavefront's diagonal; kq is its key
// minus the first query row of the current tile, and P is zeroed where the
// key follows the query.  BAND (with MASK): P is also zeroed where the query
// lies more than win rows after the key (outside a sliding window).
template <bool MASK, bool BAND = false>
__device__ __forceinline__ void dkdv_step(const uint32_t (&na)[8], int rowN,
                                          const uint32_t (&ta)[4][2], int rowC,
                                          const uint32_t (&nn)[8], uint32_t ini_nn,
                                          const bf16x8 (&kreg)[8], const bf16x8 (&vreg)[8],
                                          bf16x8 (&pre)[8], f32x16& s_cur, f32x16& p_cur,
                                          f32x16& s_nxt, f32x16& p_nxt, f32x16 (&dka)[4],
                                          f32x16 (&dva)[4], int lane, int kq, u16* ds_blk,
                                          int win = 0) {
  const int half = lane >> 5;
  const uint32_t rc = rowC * 256;
  // element r of the current block: query row r0 + 16 (r/8) + r%8; round i
  // handles elements 2i, 2i+1 (rows rr(i), rr(i) + 1)
  const int r0 = rowC + 8 * half;
  auto rr = [&](int i) { return r0 + 16 * (i >> 2) + 2 * (i & 3); };
  bf16x8 aq[4], ag[4];  // row operands of rounds 4..7
  bf16x8 bg[2][4], bq[2][4];
  // transposed operands of chunk j, block db: dout^T (bg) and Q^T (bq)
  auto tr_read = [&](int j, int db, bool dq) {
    if (dq)
      bq[j][db] = tr_operand(ta[db], rc + j * 16 * 256);
    else
      bg[j][db] = tr_operand(ta[db], rc + j * 16 * 256 + TILE_B);
  };
  uint32_t pw[8], sw[8];  // bf16 pairs (elements 2i, 2i+1)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < 4) read_rows(na, rowN, i + 4, aq[i], ag[i]);
    tr_read(0, i >> 1, i & 1);
    mfma_chain_first_or_next(i, s_nxt, i < 4 ? pre[i] : aq[i - 4], kreg[i]);
    const int r = 2 * i;
    float p0 = fast_exp2(s_cur[r]);
    float p1 = fast_exp2(s_cur[r + 1]);
    if (MASK) {  // rows rr(i), rr(i) + 1 of the current tile
      if (kq > rr(i) || (BAND && rr(i) - kq > win)) p0 = 0.f;
      if (kq > rr(i) + 1 || (BAND && rr(i) + 1 - kq > win)) p1 = 0.f;
    }
    pw[i] = pack_bf16x2(p0, p1);
    sw[i] = pack_bf16x2(p0 * p_cur[r], p1 * p_cur[r + 1]);
    // keep this round's VALU work in this round (no sinking to the first use)
    asm volatile("" : "+v"(pw[i]), "+v"(sw[i]));
    mfma_chain_first_or_next(i, p_nxt, i < 4 ? pre[4 + i] : ag[i - 4], vreg[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const bf16x8 pb[2] = {as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3])),
                        as_bf16x8(make_uint4(pw[4], pw[5], pw[6], pw[7]))};
  const bf16x8 sb[2] = {as_bf16x8(make_uint4(sw[0], sw[1], sw[2], sw[3])),
                        as_bf16x8(make_uint4(sw[4], sw[5], sw[6], sw[7]))};
  if (ds_blk) store_ds(ds_blk, sb, lane);
  // dV += P^T dout, dK += dS^T Q for the current block
  const uint32_t ia = ini_nn + 4 * (rowC + 8 * half);  // load_chain_init's rows
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int j = m >> 3, db = (m >> 1) & 3;
    if (m & 1)
      mfma_acc(dka[db], bq[j][db], sb[j]);
    else
      mfma_acc(dva[db], bg[j][db], pb[j]);
    if (m < 8) {
      tr_read(1, m >> 1, m & 1);  // chunk 1, eight MFMAs ahead
    } else {
      // the block two ahead: initial values first (needed by its first MFMA)
      const int x = m - 8;
      if (x < 4) {
        const uint32_t o = (x & 1) * 16 + (x >> 1) * 64;
        const uint4 sv = lds_ld16(ia + o), pv = lds_ld16(ia + o + 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s_cur[4 * x + e] = __uint_as_float((&sv.x)[e]);
          p_cur[4 * x + e] = __uint_as_float((&pv.x)[e]);
        }
      } else {
        read_rows(nn, rowC, x - 4, pre[x - 4], pre[x]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The rows of a tile's lse and delta (raw, in the shared buffer) rewritten
// into this wavefront's own copy as -lse log2(e) and -delta: the initial
// values of the score chains.  Each wavefront reads only its own copy, so no
// barrier is needed between the rewrite and the reads.
__device__ __forceinline__ void rewrite_rows(const float* raw, float* own, int lane) {
  own[lane] = raw[lane] * -kLog2e;
  own[64 + lane] = -raw[64 + lane];
}

// WIN: sliding window, key j visible to query i iff i - win <= j <= i.
// GRP: Hk key/value heads (H a multiple of Hk): a work item holds the keys of
// one key/value head, and its query tiles run over the G = H / Hk query heads
// that read it, so that dK and dV sum the group in registers (GRP = false:
// Hk = H, G = 1, and the head bookkeeping compiles away).
// ROPE: dk is written as the gradient of the raw keys (RopeBwd).
// GATE: dve and dg are written next to dv (GateBwd).
template <bool WIN, bool GRP, bool ROPE, bool GATE = false>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    u16* __restrict__ dk, u16* __restrict__ dv, u16* __restrict__ dsw, int nbt, int B, int T,
    int H, int Hk, float c_log2, float scale, int win, RopeBwd ra, GateBwd gt) {
  // NBUF query tiles (q and dout, swizzled, see tile_swz) and their lse, delta rows
  __shared__ __attribute__((aligned(1024))) char qtiles[NBUF * BUF_B];
  __shared__ __attribute__((aligned(1024))) char kstage[2 * TILE_B];  // K rows of an item
  __shared__ __attribute__((aligned(16))) float lsd[NBUF][2][QT_ROWS];
  // each wavefront's rewritten lse, delta rows (rewrite_rows) per buffer
  __shared__ __attribute__((aligned(16))) float lsw[4][NBUF][2][QT_ROWS];
  __shared__ __attribute__((aligned(1024))) char estage[4][4096];  // dK, dV rows on the way out

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int G = GRP ? H / Hk : 1;
  const int n_ktiles = (T + KT_KEYS - 1) / KT_KEYS;
  const int n_items = B * Hk * n_ktiles;
  const int n_qt = (T + QT_ROWS - 1) / QT_ROWS;
  // 32-bit row offsets within one batch (T * H * D < 2^31 is checked on the host)
  const int rs = H * D;    // q, dout rows
  const int rsk = Hk * D;  // k, v, dk, dv rows
  const uint32_t rsb = static_cast<uint32_t>(rs) * 2;    // bytes between rows
  const uint32_t rsbk = static_cast<uint32_t>(rsk) * 2;
  const uint32_t qoff = tile_copy_offset(wave, lane, rsb);
  const uint32_t koff = tile_copy_offset(wave, lane, rsbk);
  const TileOffsets ofs = tile_operand_offsets(lane);
  const uint32_t qt_lds = lds_addr(qtiles);
  const uint32_t lsd_lds = lds_addr(&lsd[0][0][0]);
  const uint32_t kst_lds = lds_addr(kstage);
  const uint32_t est_lds = lds_addr(&estage[wave][0]);
  // init rows of the score chains for buffer u (load_chain_init)
  const uint32_t lsw_lds = lds_addr(&lsw[wave][0][0][0]);
  auto ini = [&](int u) { return lsw_lds + static_cast<uint32_t>(u) * 2 * QT_ROWS * 4; };
  auto rewrite = [&](int u) { rewrite_rows(&lsd[u][0][0], &lsw[wave][u][0][0], lane); };

  // A work item: the 128-key tile k0 / 128 of key/value head hk of batch b
  // (xcd_tile_map_grouped order, key tile 0, the one with the most work,
  // first), whose keys are seen by the query tiles qt0 .. qte - 1 of each of
  // the G query heads hk G .. hk G + G - 1: N = G (qte - qt0) query tiles,
  // position n = g (qte - qt0) + (t - qt0) for query head hk G + g, tile t.
  struct Item {
    int b, hk, k0, qt0, qte, N;
    size_t kbase, qbase;  // k/v rows of head hk, q/dout rows of head hk G
    size_t lbase;         // lse/delta row of head hk G
  };
  auto item_at = [&](int r, Item& it) -> bool {
    const int vb = persistent_item(r);
    if (vb >= n_items) return false;
    int bhk, kt;
    xcd_tile_map_grouped(vb, B * Hk, n_ktiles, kHeadGroup, bhk, kt);
    it.b = bhk / Hk;
    it.hk = bhk % Hk;
    it.k0 = kt * KT_KEYS;
    it.qt0 = it.k0 / QT_ROWS;
    it.qte = WIN ? min(n_qt, (it.k0 + KT_KEYS - 1 + win) / QT_ROWS + 1) : n_qt;
    it.N = G * (it.qte - it.qt0);
    it.kbase = static_cast<size_t>(it.b) * T * rsk + static_cast<size_t>(it.hk) * D;
    it.qbase = static_cast<size_t>(it.b) * T * rs + static_cast<size_t>(it.hk) * G * D;
    it.lbase = (static_cast<size_t>(it.b) * H + static_cast<size_t>(it.hk) * G) * T;
    return true;
  };

  // Query tile qt of query head h (of item it's batch) -> buffer u (see
  // copy_tile); wavefronts 0 and 1 also copy its lse and delta rows.  Rows
  // past T are past the end of the buffer range and arrive as zeros: a zero
  // query row with zero dout, lse and delta adds nothing to dK or dV.
  // qh, lh: offsets of the query head's row 0 in q / dout and in lse / delta.
  auto issue_at = [&](size_t qh, size_t lh, int qt, int u) {
    const int q0 = qt * QT_ROWS;
    const uint32_t nrec = static_cast<uint32_t>(T - q0) * rsb;
    const size_t off = qh + static_cast<size_t>(q0 * rs);
    copy_tile(buffer_rsrc(q + off, nrec), qoff, rsb, qt_lds + u * BUF_B, wave);
    copy_tile(buffer_rsrc(dout + off, nrec), qoff, rsb, qt_lds + u * BUF_B + TILE_B, wave);
    const size_t row0 = lh + static_cast<size_t>(q0);
    if (wave == 0)
      dma4(buffer_rsrc(lse + row0, static_cast<uint32_t>(T - q0) * 4), 4 * lane,
           lsd_lds + u * 512);
    if (wave == 1)
      dma4(buffer_rsrc(delta + row0, static_cast<uint32_t>(T - q0) * 4), 4 * lane,
           lsd_lds + u * 512 + 256);
  };
  auto issue_tile = [&](const Item& it, int g, int qt, int u) {  // query head hk G + g
    issue_at(it.qbase + static_cast<size_t>(g * D), it.lbase + static_cast<size_t>(g * T), qt,
             u);
  };
  // The tile at position n of item it -> buffer u (n < it.N; a division, so
  // only outside the steady loop).
  auto issue = [&](const Item& it, int n, int u) {
    const int nt = it.qte - it.qt0;
    issue_tile(it, n / nt, it.qt0 + n % nt, u);
  };
  // The 128 K (or V) rows of item it -> LDS at dst (two swizzled 64-row tiles).
  // Keys past T arrive as zeros: their gradients are never stored and, since
  // every real query precedes them, the causal mask removes them from every
  // real query's dS.
  auto copy_rows = [&](const Item& it, const u16* src, uint32_t dst) {
    const int nk = T - it.k0;  // >= 1
    const uint32_t n0 = static_cast<uint32_t>(min(nk, 64)) * rsbk;
    const uint32_t n1 = static_cast<uint32_t>(max(nk - 64, 0)) * rsbk;
    const size_t off0 = it.kbase + static_cast<size_t>(it.k0) * rsk;
    copy_tile<4, (NA_NT_EXTRA & 8) != 0>(buffer_rsrc(src + off0, n0), koff, rsbk, dst, wave);
    copy_tile<4, (NA_NT_EXTRA & 8) != 0>(
        buffer_rsrc(src + off0 + static_cast<size_t>(64) * rsk, n1), koff, rsbk, dst + TILE_B,
        wave);
  };
  // Every copy issued so far has landed and every wavefront is past its
  // reads of the buffer that the next copy overwrites.
  auto sync_tiles = [&]() {
    wait_vmem();
    wait_lds();
    __syncthreads();
  };

  // The query tiles of the items form one stream through the NBUF buffers:
  // the item whose first tile sits in buffer gb has the tile at position n in
  // buffer (gb + n) % NBUF, and the next item's first tiles follow on.  The
  // copies of the next item's K rows, of its first two query tiles and (once
  // the last tile is done) of its V rows overlap the end of the current item,
  // so only the register reads of K and V remain between two items.
  Item cur, nxt;
  if (!item_at(0, cur)) return;
  bool has_next = item_at(1, nxt);
  int gb = 0;
  copy_rows(cur, k, kst_lds);
  copy_rows(cur, v, qt_lds + 2 * BUF_B);
  issue(cur, 0, 0);
  if (1 < cur.N) issue(cur, 1, 1);
  sync_tiles();

  for (int r = 0;; ++r) {
    // K rows in kstage, V rows in buffer (gb + 2) % NBUF, the tiles at
    // positions 0 and 1 in buffers gb, gb + 1: all landed.
    const int qt0 = cur.qt0;
    const int qte = cur.qte;
    const int nt = qte - qt0;  // query tiles of this item per query head
    const int N = cur.N;
    const int kw0 = cur.k0 + 32 * wave;
    const size_t kbase = cur.kbase;
    const int ub2 = gb == 0 ? 2 : gb - 1;  // (gb + 2) % NBUF
    // The score chains start from -lse log2(e) and -delta: every wavefront
    // rewrites the rows of the tiles at positions 0 and 1 into its own copy
    // (and of position n + 1 at each later tile's barrier).
    rewrite(gb);
    if (1 < N) rewrite((gb + 1) % NBUF);
    // K^T and V^T operands: lane holds row kw0 + l32, elements 16 kc + 8 half
    // + 0..7, read from the rows staged with 16 lanes per row.
    const int krow = kw0 + l32;
    bf16x8 kreg[8], vreg[8];
    {
      const int rr = 32 * (wave & 1) + l32;  // row within the 64-row half
      const uint32_t o_row = (wave >> 1) * TILE_B + rr * 256;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const uint32_t o = o_row + 16 * ((2 * kc + half) ^ tile_swz(rr));
        // K' = s log2(e) K, rounded to bf16: the S chain then holds the
        // exponent of P in the exp2 domain directly
        const uint4 kw = lds_ld16(kst_lds + o);
        const uint32_t w[4] = {kw.x, kw.y, kw.z, kw.w};
        uint32_t ks[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ks[j] = pack_bf16x2(__uint_as_float(w[j] << 16) * c_log2,
                              __uint_as_float(w[j] & 0xffff0000u) * c_log2);
        // moved into AGPRs here, once per item (defined by this asm in the
        // AGPR class, so the MFMAs find it there without a copy per use)
        asm volatile("" : "=a"(kreg[kc]) : "0"(as_bf16x8(make_uint4(ks[0], ks[1], ks[2], ks[3]))));
        vreg[kc] = as_bf16x8(lds_ld16(qt_lds + ub2 * BUF_B + o));
      }
    }
    wait_lds();
    __syncthreads();  // kstage and buffer (gb + 2) % NBUF are free again
    if (2 < N) issue(cur, 2, ub2);
    int nx = 0;              // leading query tiles of the next item issued
    bool k_next = false;     // next item's K rows issued

    f32x16 dka[4], dva[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dka[i] = f32x16{};
      dva[i] = f32x16{};
    }

    // dS blocks of this wavefront's 32 keys for query head h (when a dS
    // workspace is given).  Only blocks with a query row < T exist in the
    // packed layout; a block made of padding rows only (the tail of the last
    // tile) is not stored.  Stored blocks always have kblk <= qblk.
    const int kblk = kw0 / 32;
    auto ds_of = [&](int h, int qblk) -> u16* {
      return (dsw && 32 * qblk < T)
                 ? dsw + ds_block_index(cur.b * H + h, nbt, qblk, kblk)
                 : nullptr;
    };

    // One software pipeline over the 32-query blocks from the diagonal on:
    // the step for block j computes the probabilities of j, the scores of j+1
    // and the dK/dV update of j.  This wavefront's first block of each query
    // head is its diagonal block bw (masked); blocks before it hold no visible
    // (query, key) pair and are skipped, and the slot of block bw - 1 computes
    // bw's scores.  Tile t holds blocks 2t, 2t+1; block 2t+1's step reads the
    // scores of the next block from the tile at the next position (the next
    // query head's first tile after a head's last one, whose scores are the
    // ones its diagonal block needs).  At the sync before position n (n > 0)
    // position n+1 has landed and position n-1's buffer is free for the copy
    // of position n+2.  After the last position the second step still
    // computes scores of a block past the end (from whatever the next buffer
    // holds); they are never used.
    const int bw = kw0 / 32;
    f32x16 s0, p0, s1, p1;  // scores of even blocks in s0/p0, of odd blocks in s1/p1
    uint32_t nc[8];         // row-read addresses of the current tile
    nat_addr(qt_lds + gb * BUF_B, ofs, nc);
    bf16x8 pre[8];          // first row operands of the next block's chains
    if (bw == 2 * qt0)  // block 0 of position 0 is the diagonal
      dkdv_scores(nc, 0, ini(gb), nc, 32, ini(gb), kreg, vreg, s0, p0, s1, p1, pre, lane);
    int u = gb;  // buffer of the current position
    // The first two tiles of each query head (every diagonal block of the
    // workgroup) take the per-wavefront branches; the rest run one branch-free
    // body.
    auto tile = [&](int g, size_t qh, size_t lh, int n, int t, auto steady) {
      const int h = cur.hk * G + g;  // query head; qh, lh: its row-0 offsets
      constexpr bool STEADY = decltype(steady)::value;
      const int un = u == NBUF - 1 ? 0 : u + 1;  // buffer of position n + 1
      if (n > 0) {
        sync_tiles();
        const int u2 = un == NBUF - 1 ? 0 : un + 1;
        const int pos = n + 2;
        if (pos < N) {
          // position n + 2: tile t + 2 of query head g, else of a later head
          // (two heads on when a head has a single tile); no division
          if (!GRP || t + 2 < qte) {
            issue_at(qh, lh, t + 2, u2);
          } else {
            int g2 = g + 1, t2 = t + 2 - nt;
            if (t2 >= qte) t2 -= nt, ++g2;
            issue_tile(cur, g2, t2, u2);
          }
        } else if (has_next && pos - N == nx && nx < 2 && nx < nxt.N) {
          issue(nxt, nx, u2);  // the next item's position nx, in stream order
          ++nx;
        }
        if (n == N - 1 && has_next) {
          copy_rows(nxt, k, kst_lds);
          k_next = true;
        }
        if (n + 1 < N) rewrite(un);  // position n+1 (landed at this barrier)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      uint32_t tc[4][2], nn[8];
      tr_addr(qt_lds + u * BUF_B, ofs, tc);
      nat_addr(qt_lds + un * BUF_B, ofs, nn);
      const int kq = krow - QT_ROWS * t;
      const int j0 = 2 * t, j1 = 2 * t + 1;
      // with a window: some row of tile t lies past the window of this
      // wavefront's first key, so its steps also take the band select
      const bool edge = WIN && QT_ROWS * t + QT_ROWS - 1 - kw0 > win;
      // the block two ahead of each step: the same rows of the next position
      const uint32_t inn = ini(un);
      // with a window, a block whose first query row is more than win past
      // this wavefront's last key holds no visible pair, nor does any later
      // block of the item: the wavefront skips their steps (and their dS
      // blocks, which the dQ GEMM never reads) but keeps taking part in the
      // copies and barriers
      const bool gone0 = WIN && 32 * j0 - (kw0 + 31) > win;
      const bool gone1 = WIN && 32 * j1 - (kw0 + 31) > win;
      // block j0 (rows 0..31 of tile t), scores of rows 32..63
      if (gone0) {
      } else if (STEADY || j0 > bw) {
        if (WIN && edge)
          dkdv_step<true, true>(nc, 32, tc, 0, nn, inn, kreg, vreg, pre, s0, p0, s1, p1, dka, dva,
                                lane, kq, ds_of(h, j0), win);
        else
          dkdv_step<false>(nc, 32, tc, 0, nn, inn, kreg, vreg, pre, s0, p0, s1, p1, dka, dva, lane,
                           kq, ds_of(h, j0));
      } else if (j0 == bw) {
        dkdv_step<true, WIN>(nc, 32, tc, 0, nn, inn, kreg, vreg, pre, s0, p0, s1, p1, dka, dva,
                             lane, kq, ds_of(h, j0), win);
      } else if (j0 == bw - 1) {  // rows 32..63 hold the diagonal
        dkdv_scores(nc, 32, ini(u), nn, 0, inn, kreg, vreg, s1, p1, s0, p0, pre, lane);
      }
      // block j1 (rows 32..63 of tile t), scores of the next position's rows 0..31
      if (gone1) {
        // the next query head's first block is this wavefront's diagonal
        // (wavefront 0): its scores come from this slot, as in the step
        if (GRP && t == qte - 1 && g + 1 < G && bw == 2 * qt0)
          dkdv_scores(nn, 0, inn, nn, 32, inn, kreg, vreg, s0, p0, s1, p1, pre, lane);
      } else if (STEADY || j1 > bw) {
        if (WIN && edge)
          dkdv_step<true, true>(nn, 0, tc, 32, nn, inn, kreg, vreg, pre, s1, p1, s0, p0, dka, dva,
                                lane, kq, ds_of(h, j1), win);
        else
          dkdv_step<false>(nn, 0, tc, 32, nn, inn, kreg, vreg, pre, s1, p1, s0, p0, dka, dva, lane,
                           kq, ds_of(h, j1));
      } else if (j1 == bw) {
        dkdv_step<true, WIN>(nn, 0, tc, 32, nn, inn, kreg, vreg, pre, s1, p1, s0, p0, dka, dva,
                             lane, kq, ds_of(h, j1), win);
      } else if (j1 == bw - 1) {  // the next position's rows 0..31 hold the diagonal
        dkdv_scores(nn, 0, inn, nn, 32, inn, kreg, vreg, s0, p0, s1, p1, pre, lane);
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) nc[kc] = nn[kc];
      u = un;
    };
    const int t_diag_end = min(qt0 + 2, qte);
    for (int g = 0; g < G; ++g) {
      const int n0 = g * nt - qt0;  // position of tile t: n0 + t
      const size_t qh = cur.qbase + static_cast<size_t>(g * D);
      const size_t lh = cur.lbase + static_cast<size_t>(g * T);
      for (int t = qt0; t < t_diag_end; ++t) tile(g, qh, lh, n0 + t, t, std::false_type{});
      for (int t = t_diag_end; t < qte; ++t) tile(g, qh, lh, n0 + t, t, std::true_type{});
    }

    // Every wavefront is done with the last tile's buffer: the next item's V
    // rows go there, and whatever the stream has not copied yet of its K rows
    // and first two query tiles follows (issue_next).
    mfma_drain(dka, dva);
    wait_lds();
    __syncthreads();
    const int ulast = (gb + N - 1) % NBUF;
    auto issue_next = [&]() {
      if (has_next) {
        if (!k_next) copy_rows(nxt, k, kst_lds);
        copy_rows(nxt, v, qt_lds + ulast * BUF_B);
        for (int j = nx; j < 2; ++j)
          if (j < nxt.N) issue(nxt, j, (gb + N + j) % NBUF);
      }
    };

    // dka[db], dva[db] (dK^T, dV^T blocks) element r: key kw0 + l32,
    // d = 32 db + 8 (r/4) + 4 half + r%4.  The rows leave through this
    // wavefront's 4 KiB of LDS, 16 rows at a time, so that 16 lanes store one
    // 256-byte row: stored straight from registers, every lane would write 8
    // bytes to a different row.  Staging rows are swizzled by 16-byte chunk
    // (chunk c of row r at c ^ r).  Only this wavefront touches its staging
    // area, so no barrier is needed between the rounds; but the previous
    // round's reads must be done before a round overwrites the rows, which the
    // compiler does not see (it may sink a read into the conditional store
    // that uses it, past the next round's writes): each round starts with an
    // LDS wait that is also a compiler memory barrier.
    // Round sh of acc (scaled by sc): lane i gets chunk c = i % 16 of the row
    // of key key_of(sh, m) in x[m].  (The lane index is passed through an
    // empty asm so that what derives from it is computed here, not kept live
    // through the loop above, which needs every register.)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int c = ln & 15;
    auto key_of = [&](int sh, int m) { return kw0 + 16 * sh + 4 * m + (ln >> 4); };
    auto stage_round = [&](const f32x16* acc, float sc, int sh, uint4 (&x)[4]) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (((ln & 31) >> 4) == sh) {
        const int rr = ln & 15;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int e = 4 * g;
            lds_st8(est_lds + rr * 256 + 16 * ((4 * db + g) ^ rr) + 8 * (ln >> 5),
                    pack_bf16x2(acc[db][e] * sc, acc[db][e + 1] * sc),
                    pack_bf16x2(acc[db][e + 2] * sc, acc[db][e + 3] * sc));
          }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int rr = 4 * m + (ln >> 4);
        x[m] = lds_ld16(est_lds + rr * 256 + 16 * (c ^ rr));
      }
    };
    auto store_round = [&](u16* dst, int sh, const uint4 (&x)[4]) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int key = key_of(sh, m);
#if NA_NT_EXTRA & 4
        if (key < T) st16_nt(dst + kbase + key * rsk + 8 * c, x[m]);
#else
        if (key < T) st16(dst + kbase + key * rsk + 8 * c, x[m]);
#endif
      }
    };

    if constexpr (!ROPE) {
      issue_next();
#pragma unroll
      for (int tsel = 0; tsel < 2; ++tsel)  // dK, then dV
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          uint4 x[4];
          stage_round(tsel ? dva : dka, tsel ? 1.f : scale, sh, x);
          store_round(tsel ? dv : dk, sh, x);
        }
    } else {
      // ROPE (and GATE): the rounds need global loads (raw key chunks with
      // their angles; ve chunks and gate logits).  Vector memory operations
      // retire in issue order, and the copies of issue_next are asm the
      // compiler does not count, so a load issued behind a store or a copy
      // would wait for them as well: each round's loads are issued before the
      // previous round's stores, and issue_next follows the last of them.
      auto rope_load = [&](int sh, int m) {
        const int kr = min(key_of(sh, m), T - 1);
        return rope_row_load(ra.raw + kbase + kr * rsk + 8 * c, ra, kr, c);
      };
      RopeRow rrow[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) rrow[m] = rope_load(0, m);
      uint4 x0[4], x1[4];
      stage_round(dka, scale, 0, x0);
#pragma unroll
      for (int m = 0; m < 4; ++m) x0[m] = rope_bwd_chunk(x0[m], rrow[m], ra.eps, c);
#pragma unroll
      for (int m = 0; m < 4; ++m) rrow[m] = rope_load(1, m);
      store_round(dk, 0, x0);
      stage_round(dka, scale, 1, x1);
#pragma unroll
      for (int m = 0; m < 4; ++m) x1[m] = rope_bwd_chunk(x1[m], rrow[m], ra.eps, c);
      // GATE: the ve chunks and gate logits of the dV rows, loaded once the
      // angles' registers are free; waited for (all but the 4 stores behind
      // them) before the copies, which the wait would otherwise include
      const size_t gbase = static_cast<size_t>(cur.b) * T * Hk + cur.hk;  // gate row of key 0
      uint4 vev[GATE ? 8 : 1];
      float glv[GATE ? 8 : 1];
      if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kr = min(key_of(i >> 2, i & 3), T - 1);
          vev[i] = ld16(gt.ve + kbase + kr * rsk + 8 * c);
          glv[i] = bf16_to_f32(gt.gate[gbase + static_cast<size_t>(kr) * Hk]);
        }
      }
      store_round(dk, 1, x1);
      if constexpr (GATE) wait_vmem_but<4>();
      issue_next();
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        uint4 x[4];
        stage_round(dva, 1.f, sh, x);
        store_round(dv, sh, x);
        if constexpr (GATE) {  // dv' chunks -> dve chunks and (lane c = 0) dg
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int key = key_of(sh, m), i = GATE ? 4 * sh + m : 0;
            const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-glv[i] * kLog2e));
            float xv[8], ev[8], y[8];
            unpack8(x[m], xv);
            unpack8(vev[i], ev);
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              y[j] = 3.f * sg * xv[j];
              dot = fmaf(ev[j], xv[j], dot);
            }
            dot = sum16(dot);
            if (key < T) {
              st16(gt.dve + kbase + key * rsk + 8 * c, pack8(y));
              if (c == 0)
                gt.dgate[gbase + static_cast<size_t>(key) * Hk] =
                    __builtin_bit_cast(u16, to_bf16(3.f * sg * (1.f - sg) * dot));
            }
          }
        }
      }
    }

    if (!has_next) break;
    sync_tiles();  // the next item's K, V rows and first query tiles have landed
    gb = (gb + N) % NBUF;
    cur = nxt;
    has_next = item_at(r + 2, nxt);
  }
}

// ---------------------------------------------------------------- dQ

constexpr int DQ_ROWS = 128;  // queries per workgroup (32 per wavefront)
constexpr int RS = D + 8;     // row-major tile stride (bf16 elements)
constexpr int DQ_KEYS = 64;   // keys per LDS tile

// One 32-key block of a dQ step for one wavefront (32 queries), in three
// phases:
//   scores:  S^T = K Q^T, dP^T = V dout^T  (A = K / V rows from LDS, B = Q /
//            dout in registers; lane: query, element r: key acc_row(lane, r))
//   probs:   P = exp2(c S - lse2), dS = P (dP - delta), rounded to bf16
//   accum:   dQ^T += K^T dS^T  (A = transposed K tile, B = dS^T from registers)
__device__ __forceinline__ void dq_scores(const u16* Ks, const u16* Vs, int row0,
                                          const bf16x8 (&qreg)[8], const bf16x8 (&greg)[8],
                                          f32x16& sacc, f32x16& pacc, int lane) {
  const int half = lane >> 5;
  const int l32 = lane & 31;
  sacc = f32x16{};
  pacc = f32x16{};
  const u16* kp = &Ks[(row0 + perm_row(l32)) * RS + 8 * half];
  const u16* vp = &Vs[(row0 + perm_row(l32)) * RS + 8 * half];
#pragma unroll
  for (int k4 = 0; k4 < 8; k4 += 4) {
    bf16x8 ak[4], av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ak[i] = as_bf16x8(ld16(kp + 16 * (k4 + i)));
      av[i] = as_bf16x8(ld16(vp + 16 * (k4 + i)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sacc = mfma32(ak[i], qreg[k4 + i], sacc);
      pacc = mfma32(av[i], greg[k4 + i], pacc);
    }
  }
}

// MASK: keys after the query are dropped; BAND: so are keys more than win
// before it (sliding window).
template <bool MASK, bool BAND = false>
__device__ __forceinline__ void dq_probs(const f32x16& sacc, const f32x16& pacc, bf16x8 (&sb)[2],
                                         int lane, int qrow_minus_k0, int row0, float lse2,
                                         float dl, float c_log2, int win = 0) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float p = fast_exp2(fmaf(sacc[r], c_log2, -lse2));
    const int d = qrow_minus_k0 - (row0 + acc_row(lane, r));  // query - key
    if (MASK && d < 0) p = 0.f;                               // key after query
    if (BAND && d > win) p = 0.f;                             // key before the window
    sb[r >> 3][r & 7] = to_bf16(p * (pacc[r] - dl));
  }
}

__device__ __forceinline__ void dq_accum(const bf16x8 (&sb)[2], const u16* Kt, int row0,
                                         f32x16 (&dqa)[4], int lane) {
  const int half = lane >> 5;
  const int l32 = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cg = row0 / 8 + 2 * j + half;  // keys row0 + 16 j + 8 half + 0..7
    bf16x8 a[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) a[db] = as_bf16x8(ld16(&Kt[toff(db * 32 + l32, cg)]));
#pragma unroll
    for (int db = 0; db < 4; ++db) dqa[db] = mfma32(a[db], sb[j], dqa[db]);
  }
}

template <bool MASK, bool BAND = false>
__device__ __forceinline__ void dq_block(const u16* Ks, const u16* Vs, const u16* Kt,
                                         const bf16x8 (&qreg)[8], const bf16x8 (&greg)[8],
                                         f32x16 (&dqa)[4], int kb, int lane, int qrow_minus_k0,
                                         float lse2, float dl, float c_log2, int win = 0) {
  f32x16 sacc, pacc;
  dq_scores(Ks, Vs, 32 * kb, qreg, greg, sacc, pacc, lane);
  bf16x8 sb[2];
  dq_probs<MASK, BAND>(sacc, pacc, sb, lane, qrow_minus_k0, 32 * kb, lse2, dl, c_log2, win);
  dq_accum(sb, Kt, 32 * kb, dqa, lane);
}

// Steady-state step: probabilities of the current block, scores of the next
// block, the current block's dQ update; one basic block.
__device__ __forceinline__ void dq_step(const u16* KsN, const u16* VsN, int rowN, const u16* Kt,
                                        int rowC, const bf16x8 (&qreg)[8],
                                        const bf16x8 (&greg)[8], const f32x16& s_cur,
                                        const f32x16& p_cur, f32x16& s_nxt, f32x16& p_nxt,
                                        f32x16 (&dqa)[4], int lane, float lse2, float dl,
                                        float c_log2) {
  bf16x8 sb[2];
  dq_probs<false>(s_cur, p_cur, sb, lane, 0, rowC, lse2, dl, c_log2);
  dq_scores(KsN, VsN, rowN, qreg, greg, s_nxt, p_nxt, lane);
  dq_accum(sb, Kt, rowC, dqa, lane);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS read
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // TRANS
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
  }
}

// WIN: sliding window (key j visible to query i iff i - win <= j <= i).  The
// windowed pass skips the pipelined steady part and runs every key tile from
// the first one any row of the workgroup sees through the per-tile loop, each
// block with the causal and band selects (this is the path for callers
// without a dS workspace; the GEMM over stored dS is the fast one).
template <bool WIN>
__global__ __launch_bounds__(256, 1) void dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    u16* __restrict__ dq, int B, int T, int H, int Hk, float c_log2, float scale, int win) {
  __shared__ __attribute__((aligned(16))) u16 Ks[2][DQ_KEYS * RS];
  __shared__ __attribute__((aligned(16))) u16 Vs[2][DQ_KEYS * RS];
  __shared__ __attribute__((aligned(16))) u16 Kt[2][D * DQ_KEYS];  // transposed, swizzled

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int G = H / Hk;  // query heads per key/value head, grouped on one XCD
  const int n_qt = (T + DQ_ROWS - 1) / DQ_ROWS;
  int bhk, tg;
  xcd_tile_map_grouped(static_cast<int>(blockIdx.x), B * Hk, n_qt * G, kHeadGroup, bhk, tg);
  const int qt = n_qt - 1 - tg / G;  // heaviest (last) query tile first
  const int b = bhk / Hk, hk = bhk % Hk;
  const int h = hk * G + tg % G;
  const int bh = b * H + h;
  const int q0 = qt * DQ_ROWS;
  const int qw0 = q0 + 32 * wave;
  const int rs = H * D;    // 32-bit row offsets within one batch: q, dout, dq
  const int rsk = Hk * D;  // k, v
  const size_t base = static_cast<size_t>(b) * T * rs + static_cast<size_t>(h) * D;
  const size_t kbase = static_cast<size_t>(b) * T * rsk + static_cast<size_t>(hk) * D;

  // rows past T read row T-1 (their dq is never stored)
  const int qrow = qw0 + l32;
  const int qr = min(qrow, T - 1);
  bf16x8 qreg[8], greg[8];
  {
    const size_t off = base + qr * rs + 8 * half;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      qreg[kc] = as_bf16x8(ld16(q + off + 16 * kc));
      greg[kc] = as_bf16x8(ld16(dout + off + 16 * kc));
    }
  }
  const float lse2 = lse[static_cast<size_t>(bh) * T + qr] * kLog2e;
  const float dl = delta[static_cast<size_t>(bh) * T + qr];

  f32x16 dqa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dqa[i] = f32x16{};

  const int last_q = min(q0 + DQ_ROWS, T) - 1;
  const int n_kt = last_q / DQ_KEYS + 1;
  const int lrow = tid >> 4;
  const int lchunk = tid & 15;
  // key rows past T read row T-1: always masked, any finite value works
  uint4 xk[4], xv[4];
  auto gload = [&](int kt) {
    const int k0 = kt * DQ_KEYS;  // rows clamp to T-1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t off = kbase + min(k0 + 4 * lrow + i, T - 1) * rsk + 8 * lchunk;
      xk[i] = ld16(k + off);
      xv[i] = ld16(v + off);
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&Ks[buf][(4 * lrow + i) * RS + 8 * lchunk], xk[i]);
      st16(&Vs[buf][(4 * lrow + i) * RS + 8 * lchunk], xv[i]);
    }
    tstore_4x8(Kt[buf], xk, lrow, lchunk);
  };

  // Steady part: key tiles entirely before every query of this workgroup
  // (no mask, no skipped block), software-pipelined over 32-key blocks as in
  // the dK/dV kernel.  The last step computes scores of one block past the
  // steady range; they are never used.
  const int ns = WIN ? max(q0 - win, 0) / DQ_KEYS : q0 / DQ_KEYS;
  if (!WIN && ns > 0) {
    int b = 0;
    gload(0);
    lstore(b);
    __syncthreads();
    gload(1);
    f32x16 s0, p0, s1, p1;
    dq_scores(Ks[b], Vs[b], 0, qreg, greg, s0, p0, lane);
    for (int t = 0; t < ns; ++t) {
      dq_step(Ks[b], Vs[b], 32, Kt[b], 0, qreg, greg, s0, p0, s1, p1, dqa, lane, lse2, dl,
              c_log2);
      __syncthreads();  // every wavefront is done with tile t-1 (buffer b^1)
      lstore(b ^ 1);
      __syncthreads();
      gload(min(t + 2, n_kt - 1));
      dq_step(Ks[b ^ 1], Vs[b ^ 1], 0, Kt[b], 32, qreg, greg, s1, p1, s0, p0, dqa, lane, lse2,
              dl, c_log2);
      b ^= 1;
    }
    __syncthreads();  // all wavefronts leave the pipelined loop before buffers are reused
  }

  // Diagonal part: the key tiles that overlap this workgroup's queries, one
  // barrier per tile, causal select where a tile crosses a wavefront's rows.
  gload(ns);
  for (int kt = ns; kt < n_kt; ++kt) {
    const int buf = (kt - ns) & 1;
    const int k0 = kt * DQ_KEYS;
    lstore(buf);
    __syncthreads();
    if (kt + 1 < n_kt) gload(kt + 1);

    if (k0 > qw0 + 31) continue;  // whole tile after this wavefront's queries
    const int qk = qrow - k0;
    if constexpr (WIN) {
      // blocks holding a visible pair of some row of this wavefront, both
      // selects applied
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kk = k0 + 32 * kb;
        if (kk <= qw0 + 31 && kk + 31 >= qw0 - win)
          dq_block<true, true>(Ks[buf], Vs[buf], Kt[buf], qreg, greg, dqa, kb, lane, qk, lse2,
                               dl, c_log2, win);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (k0 + DQ_KEYS - 1 > qw0) {  // tile crosses the diagonal
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (k0 + 32 * kb <= qw0 + 31)
          dq_block<true>(Ks[buf], Vs[buf], Kt[buf], qreg, greg, dqa, kb, lane, qk, lse2, dl,
                         c_log2);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dq_block<false>(Ks[buf], Vs[buf], Kt[buf], qreg, greg, dqa, kb, lane, qk, lse2, dl,
                        c_log2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (qrow < T) {
    u16* qp = dq + base + qrow * rs;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk = make_uint2(pack_bf16x2(dqa[db][4 * g] * scale, dqa[db][4 * g + 1] * scale),
                              pack_bf16x2(dqa[db][4 * g + 2] * scale, dqa[db][4 * g + 3] * scale));
        *reinterpret_cast<uint2*>(qp + 32 * db + 8 * g + 4 * half) = pk;
      }
  }
}

// ---------------------------------------------------------------- dQ from stored dS

// With a dS workspace the dK/dV kernel keeps dS (bf16, 32 x 32 blocks), and
// dQ = s dS K is a plain GEMM over the lower-triangular blocks instead of a
// pass that recomputes S and dP.  Per wavefront (32 queries) and 32-key block:
//   dQ^T += K^T dS^T   (A = K tile read transposed, B = dS^T)
// Both operands need eight consecutive keys per lane: K^T comes from the
// swizzled K tile with ds_read_b64_tr_b16 (as V^T in the forward), and dS^T
// from the stored block, gathered into [key][query] order in LDS by the copies
// (store_ds) and read with the same transposing instruction (lanes supplying rows key0 + i/4 at columns
// 4 (i%4) leave lane j with column query0 + j of keys key0 .. key0 + 3).  K
// tiles (by the whole workgroup) and each wavefront's dS blocks (by that
// wavefront) are copied HBM -> LDS by DMA, one barrier per key tile.  The dS
// stream is the HBM-bound part (about B*H*T^2 bytes against a few hundred
// cycles of MFMA per block), so its copies run two tiles ahead (three
// buffers); K tiles, mostly L2 hits, run one ahead (two buffers).  Eight
// wavefronts share each K tile: every byte through the compute unit's
// vector-memory path counts here, and the K copies are a third of it at four
// wavefronts (measured: 379 -> 356 us at d20 going from four to eight).
constexpr int DG_WAVES = 8;                // wavefronts per workgroup
constexpr int DG_ROWS = 32 * DG_WAVES;     // queries per workgroup (32 per wavefront)
constexpr int DG_KCOPY = 16 / DG_WAVES;    // 1-KB copies per wavefront of each K tile
constexpr int DG_KEYS = 64;   // keys per K tile
constexpr uint32_t DG_DS_B = 2 * 32 * 32 * 2;  // a wavefront's two dS blocks per key tile

// WIN: sliding window, key j visible to query i iff i - win <= j <= i.
// ROPE: dq is written as the gradient of the raw queries (RopeBwd).
template <bool WIN, bool ROPE>
__global__ __launch_bounds__(64 * DG_WAVES, 8 / DG_WAVES) void dq_gemm_kernel(const u16* __restrict__ k,
                                                         const u16* __restrict__ dsw,
                                                         u16* __restrict__ dq, int nbt, int B,
                                                         int T, int H, int Hk, float scale,
                                                         int win, RopeBwd ra) {
  __shared__ __attribute__((aligned(1024))) char ktile[2][kTileBytes];   // swizzled K
  __shared__ __attribute__((aligned(1024))) char sst[3][DG_WAVES][DG_DS_B];  // dS blocks per wave

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int gi = lane >> 4;   // 16-lane group
  const int i16 = lane & 15;

  const int G = H / Hk;  // query heads per key/value head, grouped on one XCD
  const int n_qt = (T + DG_ROWS - 1) / DG_ROWS;
  const int n_items = B * H * n_qt;
  for (int r = 0;; ++r) {
    const int item = persistent_item(r);
    if (item >= n_items) break;
    // every wavefront is done with the previous item's LDS tiles (the next
    // copies overwrite them)
    if (r > 0) {
      wait_lds();
      __syncthreads();
    }
    int bhk, tg;
    // heads last-first: the dK/dV pass stored their dS last, so part of it
    // may still sit in the last-level cache
    xcd_tile_map_grouped(item, B * Hk, n_qt * G, kHeadGroup, bhk, tg, true);
    const int qt = n_qt - 1 - tg / G;  // heaviest (last) query tile first
    const int b = bhk / Hk, hk = bhk % Hk;
    const int h = hk * G + tg % G;
    const int bh = b * H + h;
    const int q0 = qt * DG_ROWS;
    const int qw0 = q0 + 32 * wave;
    const int qblk = qw0 / 32;
    const bool live = qw0 < T;  // wavefront has at least one real query row
    const int rs = H * D;    // dq rows
    const int rsk = Hk * D;  // k rows
    const size_t base = static_cast<size_t>(b) * T * rs + static_cast<size_t>(h) * D;
    const size_t kbase = static_cast<size_t>(b) * T * rsk + static_cast<size_t>(hk) * D;
    // this wavefront's row of dS blocks: (qblk, 0 .. qblk), 2 KiB each, contiguous
    const u16* dsrow = dsw + ds_block_index(bh, nbt, qblk, 0);

    f32x16 dqa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dqa[i] = f32x16{};

    // ROPE: raw chunk and angles of the row that lane group gi finishes in
    // round sh, step m of the epilogue: query qw0 + 16 sh + 4 m + gi
    auto rope_load = [&](int sh, int m) {
      const int qr = min(qw0 + 16 * sh + 4 * m + gi, T - 1);
      return rope_row_load(ra.raw + base + static_cast<size_t>(qr) * rs + 8 * i16, ra, qr, i16);
    };
    RopeRow rrow[ROPE ? 4 : 1];

    const int last_q = min(q0 + DG_ROWS, T) - 1;
    const int n_kt = last_q / DG_KEYS + 1;
    // first key tile that any row of the workgroup sees (0 without a window)
    const int kt_lo = WIN ? max(q0 - win, 0) / DG_KEYS : 0;

    // K^T read addresses in buffer 0 (buffer 1: + kTileBytes)
    uint32_t ktr[4][2];
    {
      const TileOffsets ofs = tile_operand_offsets(lane);
      tr_addr(lds_addr(ktile), ofs, ktr);
    }
    // dS^T reads: 16-lane group gi supplies keys 16 c + 8 half + 4 sub + i16 / 4,
    // queries 16 (gi & 1) + 4 (i16 & 3) of a block in [key][query] order
    const uint32_t st_lds = lds_addr(&sst[0][wave][0]);
    const uint32_t st_off =
        ((8 * half + (i16 >> 2)) * 32 + 16 * (gi & 1) + 4 * (i16 & 3)) * 2;
    const uint32_t rsb = static_cast<uint32_t>(rsk) * 2;
    const uint32_t kvoff = tile_copy_offset(wave, lane, rsb);
    const uint32_t kt_lds = lds_addr(ktile);
    // the wavefront's blocks of key tile kt: kblk = 2 kt, 2 kt + 1 (if <= qblk)
    const uint32_t ds_rows = static_cast<uint32_t>(qblk + 1) * 2048;  // bytes of its row
    const i32x4 ds_rsrc = buffer_rsrc(dsrow, live ? ds_rows : 0);
    // Copy j (0 .. DG_KCOPY - 1) of this wavefront's share of K tile kt / copy
    // j (0..3) of its dS blocks of key tile kt.  The copies of the next tiles are spread between the
    // current tile's MFMAs: issued in a burst they stall the issuing wavefront
    // behind the compute unit's vector-memory queue.
    auto issue_k = [&](int kt, int buf, int j) {
      const int k0 = kt * DG_KEYS;
      const uint32_t nrec = static_cast<uint32_t>(T - k0) * rsb;  // keys past T read as 0
      dma16(buffer_rsrc(k + kbase + static_cast<size_t>(k0) * rsk, nrec),
            kvoff + 4 * DG_WAVES * j * rsb,
            kt_lds + buf * kTileBytes + 1024 * (wave + DG_WAVES * j));
    };
    // LDS chunk j (0..3) of a key tile's dS: block kb = j / 2 as a [key][query]
    // matrix, keys 16 (j % 2) .. + 15; lane L writes key 16 (j % 2) + L / 4,
    // queries 8 (L % 4) .. + 7, which it gathers from the stored order
    // (store_ds: query chunk (L % 4) / 2 at 1024 bytes apart, half L % 2)
    const uint32_t ds_gather = 1024 * ((lane & 3) >> 1) + 32 * (lane >> 2) + 16 * (lane & 1);
    auto issue_ds = [&](int kt, int sbuf, int j) {
      // blocks past qblk are past the resource's end (zeros, never read)
      const uint32_t src = kt * 4096 + (j >> 1) * 2048 + (j & 1) * 512 + ds_gather;
      if constexpr ((NA_DS_NT & 1) != 0)
        dma16_nt(ds_rsrc, src, st_lds + sbuf * (DG_WAVES * DG_DS_B) + j * 1024);
      else
        dma16(ds_rsrc, src, st_lds + sbuf * (DG_WAVES * DG_DS_B) + j * 1024);
    };

    // Copies in issue order: K(0), dS(0), dS(1), then per tile t: K(t+1),
    // dS(t+2).  At tile t, K(t) and dS(t) must have landed while dS(t+1) (the
    // last 4 copies issued, if it exists) may still be in flight.
    auto tile = [&](auto bufc, int kt) {
      constexpr uint32_t BUF = decltype(bufc)::value;
      const int sb = kt % 3;
      if (kt + 1 < n_kt)
        wait_vmem_but<4>();
      else
        wait_vmem();
      wait_lds();
      __syncthreads();
      const bool more_k = kt + 1 < n_kt, more_ds = kt + 2 < n_kt;
      // Four chunks of 16 keys, j = 2 kb + c (keys 32 kb + 16 c .. + 15 of the
      // tile); chunk j+1's operands are read while chunk j's MFMAs run.
      bf16x8 a[2][4], bs[2];
      auto read = [&](int j) {
        const int kb = j >> 1, c = j & 1;
        // keys 32 kb + 16 c + 8 half + 0..7, query column l32
        const uint32_t st = st_lds + sb * (DG_WAVES * DG_DS_B) + kb * 2048 + st_off + c * 16 * 64;
        const uint2 r0 = ds_read_tr16_at(st);
        const uint2 r1 = ds_read_tr16_at(st + 4 * 64);
        bs[j & 1] = as_bf16x8(make_uint4(r0.x, r0.y, r1.x, r1.y));
#pragma unroll
        for (int db = 0; db < 4; ++db)
          a[j & 1][db] = tr_operand(ktr[db], BUF * kTileBytes + (32 * kb + 16 * c) * 256);
      };
      read(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // all of K(kt+1) before any of dS(kt+2): the wait above relies on
        // dS(kt+1)'s copies being the last four issued
        if (j < 2) {
          if (more_k) {
#pragma unroll
            for (int c = j * DG_KCOPY / 2; c < (j + 1) * DG_KCOPY / 2; ++c)
              issue_k(kt + 1, 1 - BUF, c);
          }
        } else if (more_ds) {
          issue_ds(kt + 2, (kt + 2) % 3, 2 * (j - 2));
          issue_ds(kt + 2, (kt + 2) % 3, 2 * (j - 2) + 1);
        }
        if (j + 1 < 4) read(j + 1);
        // block 2 kt + kb of this wavefront's row exists and, with a window,
        // holds a visible pair (wavefront-uniform); the dK/dV pass stored
        // every such block
        const int kblk = 2 * kt + (j >> 1);
        if (live && kblk <= qblk && (!WIN || 32 * kblk + 31 >= 32 * qblk - win)) {
#pragma unroll
          for (int db = 0; db < 4; ++db) dqa[db] = mfma32(a[j & 1][db], bs[j & 1], dqa[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

#pragma unroll
    for (int j = 0; j < DG_KCOPY; ++j) issue_k(kt_lo, 0, j);
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_ds(kt_lo, kt_lo % 3, j);
    if (kt_lo + 1 < n_kt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) issue_ds(kt_lo + 1, (kt_lo + 1) % 3, j);
    }
    for (int kt = kt_lo; kt < n_kt; kt += 2) {
      tile(std::integral_constant<uint32_t, 0>{}, kt);
      if (kt + 1 < n_kt) tile(std::integral_constant<uint32_t, 1>{}, kt + 1);
    }

    // dqa[db] element r: query qw0 + l32, d = 32 db + 8 (r / 4) + 4 half + r % 4.
    // The rows leave through this wavefront's own dS buffers of stages 0 and 1
    // (rows 0..15 and 16..31; free once its own reads of them are done, which
    // the LDS wait first establishes, also as a compiler fence), so that 16
    // lanes store one 256-byte row (chunk c of staged row r at c ^ r).
    // ROPE: the raw query rows' gradient is formed from the staged bf16
    // gradient chunk (rope_bwd_chunk); the raw chunk and angles of the first
    // four rows a lane group finishes are loaded before the staging, those of
    // the next four once the first four are used.
    if constexpr (ROPE) {
#pragma unroll
      for (int m = 0; m < 4; ++m) rrow[m] = rope_load(0, m);
    }
    constexpr uint32_t kStage = DG_WAVES * DG_DS_B;  // bytes between a wavefront's stages
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    {
      const int rr = l32 & 15;
      const uint32_t row = st_lds + (l32 >> 4) * kStage + rr * 256 + 8 * half;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = 4 * g;
          lds_st8(row + 16 * ((4 * db + g) ^ rr),
                  pack_bf16x2(dqa[db][e] * scale, dqa[db][e + 1] * scale),
                  pack_bf16x2(dqa[db][e + 2] * scale, dqa[db][e + 3] * scale));
        }
    }
    asm volatile("" ::: "memory");  // the reads below follow the writes above
    // Round sh: lane i holds chunk i % 16 of row 4 m + i / 16 in x[m].  Vector
    // memory operations retire in issue order, so round 1's loads go out
    // before round 0's stores (a load behind a store would wait for it).
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {  // queries qw0 + 16 sh .. + 15
      uint4 x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int rr = 4 * m + gi;
        x[m] = lds_ld16(st_lds + sh * kStage + rr * 256 + 16 * (i16 ^ rr));
        if constexpr (ROPE)  // whole 16-lane groups: the row is uniform over one
          x[m] = rope_bwd_chunk(x[m], rrow[ROPE ? m : 0], ra.eps, i16);
      }
      if constexpr (ROPE) {
        if (sh == 0) {
#pragma unroll
          for (int m = 0; m < 4; ++m) rrow[m] = rope_load(1, m);
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int qr = qw0 + 16 * sh + 4 * m + gi;
        if (qr < T) st16(dq + base + static_cast<size_t>(qr) * rs + 8 * i16, x[m]);
      }
    }
  }
}

}  // namespace

std::size_t bwd_workspace_bytes(int B, int T, int H) {
  const std::size_t nblk = (static_cast<std::size_t>(T) + 31) / 32;
  return static_cast<std::size_t>(B) * H * (nblk * (nblk + 1) / 2) * 1024 * sizeof(u16);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* delta, void* ws, int B, int T, int H, int Hk, int window,
                           hipStream_t s, hipEvent_t const* ev, const void* q_raw,
                           const void* k_raw, const float* cos_t, const float* sin_t, float eps,
                           const void* ve, const void* gate, void* dve, void* dgate) {
  const bool rope = q_raw != nullptr;
  const bool gated = ve != nullptr;
  if (rope && ws == nullptr) return hipErrorInvalidValue;  // checked on the host
  if (gated && !rope) return hipErrorInvalidValue;         // the gate folds with the rope only
  const GateBwd gt{static_cast<const u16*>(ve), static_cast<const u16*>(gate),
                   static_cast<u16*>(dve), static_cast<u16*>(dgate)};
  const RopeBwd rq{static_cast<const u16*>(q_raw), cos_t, sin_t, eps};
  const RopeBwd rk{static_cast<const u16*>(k_raw), cos_t, sin_t, eps};
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float c_log2 = scale * kLog2e;
  const u16* q16 = static_cast<const u16*>(q);
  const u16* k16 = static_cast<const u16*>(k);
  const u16* v16 = static_cast<const u16*>(v);
  const u16* g16 = static_cast<const u16*>(dout);
  u16* dsw = static_cast<u16*>(ws);
  const int nblk = (T + 31) / 32;
  const int nbt = nblk * (nblk + 1) / 2;
  const long rows = static_cast<long>(B) * T * H;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  e = launch(delta_kernel, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s,
             static_cast<const u16*>(o), g16, delta, B, T, H);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  const int n_kt = (T + KT_KEYS - 1) / KT_KEYS;
  const dim3 kv_grid(persistent_grid(static_cast<long>(n_kt) * B * Hk, 1));
  // a window that covers every key of every row is the plain causal case
  const bool win = window >= 0 && window < T - 1;
  const int w = win ? window : T;
  const bool grp = Hk != H;
  auto* kv_kernel =
      gated
          ? (win ? (grp ? dkdv_kernel<true, true, true, true> : dkdv_kernel<true, false, true, true>)
                 : (grp ? dkdv_kernel<false, true, true, true>
                        : dkdv_kernel<false, false, true, true>))
      : rope ? (win ? (grp ? dkdv_kernel<true, true, true> : dkdv_kernel<true, false, true>)
                    : (grp ? dkdv_kernel<false, true, true> : dkdv_kernel<false, false, true>))
             : (win ? (grp ? dkdv_kernel<true, true, false> : dkdv_kernel<true, false, false>)
                    : (grp ? dkdv_kernel<false, true, false> : dkdv_kernel<false, false, false>));
  e = launch(kv_kernel, kv_grid, dim3(256), 0, s, q16, k16,
             v16, g16, lse, static_cast<const float*>(delta), static_cast<u16*>(dk),
             static_cast<u16*>(dv), dsw, nbt, B, T, H, Hk, c_log2, scale, w, rk, gt);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 2, s)) != hipSuccess) return e;
  if (dsw != nullptr) {
    const int n_qt = (T + DG_ROWS - 1) / DG_ROWS;
    auto* dq_kern = rope ? (win ? dq_gemm_kernel<true, true> : dq_gemm_kernel<false, true>)
                         : (win ? dq_gemm_kernel<true, false> : dq_gemm_kernel<false, false>);
    e = launch(dq_kern, dim3(persistent_grid(static_cast<long>(n_qt) * B * H, 8 / DG_WAVES)),
               dim3(64 * DG_WAVES), 0, s, k16, static_cast<const u16*>(dsw),
               static_cast<u16*>(dq), nbt, B, T, H, Hk, scale, w, rq);
  } else {
    const int n_qt = (T + DQ_ROWS - 1) / DQ_ROWS;
    e = launch(win ? dq_kernel<true> : dq_kernel<false>, dim3(static_cast<unsigned>(n_qt) * B * H),
               dim3(256), 0, s, q16, k16, v16, g16, lse, static_cast<const float*>(delta),
               static_cast<u16*>(dq), B, T, H, Hk, c_log2, scale, w);
  }
  if (e != hipSuccess) return e;
  return mark(ev, 3, s);
}

}  // namespace na
