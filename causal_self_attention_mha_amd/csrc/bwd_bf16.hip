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
//   delta_kernel  rowsum(dout * o)                        (HBM bound)
//   dkdv_kernel   one workgroup per 128-key tile; K and V stay in registers
//                 as MFMA operands, query tiles of 64 stream through LDS in
//                 both row-major and transposed copies; accumulates dK, dV
//   dq_kernel     one workgroup per 128-query tile; Q, dout stay in registers,
//                 key tiles of 64 stream through LDS; accumulates dQ
// P and dS are rounded to bf16 before they enter an MFMA; everything else is
// fp32.  Each output element is written by exactly one lane, so results are
// bitwise deterministic.
#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- delta

// 16 lanes per (b, t, h) row, 16 rows per 256-thread workgroup.
__global__ __launch_bounds__(256) void delta_kernel(const u16* __restrict__ o,
                                                    const u16* __restrict__ dout,
                                                    float* __restrict__ delta, int B, int T,
                                                    int H) {
  const long row = static_cast<long>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const long n_rows = static_cast<long>(B) * T * H;
  if (row >= n_rows) return;  // whole 16-lane groups drop out together
  const int chunk = threadIdx.x & 15;
  const uint4 a = ld16(o + row * D + 8 * chunk);
  const uint4 g = ld16(dout + row * D + 8 * chunk);
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = (&a.x)[w], y = (&g.x)[w];
    acc = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
    acc = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), acc);
  }
  acc = sum16(acc);
  if (chunk == 0) {
    const int h = static_cast<int>(row % H);
    const long bt = row / H;
    const int t = static_cast<int>(bt % T);
    const int b = static_cast<int>(bt / T);
    delta[(static_cast<size_t>(b) * H + h) * T + t] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV

constexpr int KT_KEYS = 128;  // keys per workgroup (32 per wavefront)
constexpr int QT_ROWS = 64;   // queries per LDS tile
constexpr int RS = D + 8;         // row-major tile stride (bf16 elements)

// Write rows 4*lrow + i (i = 0..3) of a 64 x 128 tile, held as four 16-byte
// chunks (column chunk `chunk`), into a row-major copy and a transposed
// (swizzled, see toff) copy.
__device__ __forceinline__ void store_tile_both(u16* nat, u16* tr, const uint4 (&x)[4], int lrow,
                                                int chunk) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st16(&nat[(4 * lrow + i) * RS + 8 * chunk], x[i]);
  tstore_4x8(tr, x, lrow, chunk);
}

__global__ __launch_bounds__(256, 1) void dkdv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    u16* __restrict__ dk, u16* __restrict__ dv, int B, int T, int H, float c_log2,
    float scale) {
  __shared__ __attribute__((aligned(16))) u16 Qs[QT_ROWS * RS];
  __shared__ __attribute__((aligned(16))) u16 Gs[QT_ROWS * RS];   // dout
  __shared__ __attribute__((aligned(16))) u16 Qt[D * QT_ROWS];   // transposed, swizzled
  __shared__ __attribute__((aligned(16))) u16 Gt[D * QT_ROWS];
  __shared__ __attribute__((aligned(16))) float lse2s[QT_ROWS];
  __shared__ __attribute__((aligned(16))) float dls[QT_ROWS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int BH = B * H;
  const int kt = static_cast<int>(blockIdx.x) / BH;  // key tile 0 has the most work: first
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / H, h = bh % H;
  const int k0 = kt * KT_KEYS;
  const int kw0 = k0 + 32 * wave;
  const size_t rs = static_cast<size_t>(H) * D;
  const size_t base = static_cast<size_t>(b) * T * rs + static_cast<size_t>(h) * D;
  const float* lse_bh = lse + static_cast<size_t>(bh) * T;
  const float* del_bh = delta + static_cast<size_t>(bh) * T;

  // K^T and V^T operands of S = Q K^T and dP = dout V^T: lane holds row
  // kw0 + l32, elements 16 kc + 8 half + 0..7.
  const int krow = kw0 + l32;
  bf16x8 kreg[8], vreg[8];
  if (krow < T) {
    const u16* kp = k + base + static_cast<size_t>(krow) * rs + 8 * half;
    const u16* vp = v + base + static_cast<size_t>(krow) * rs + 8 * half;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      kreg[kc] = as_bf16x8(ld16(kp + 16 * kc));
      vreg[kc] = as_bf16x8(ld16(vp + 16 * kc));
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      kreg[kc] = as_bf16x8(make_uint4(0, 0, 0, 0));
      vreg[kc] = kreg[kc];
    }
  }

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dka[i] = f32x16{};
    dva[i] = f32x16{};
  }

  const int n_qt = (T + QT_ROWS - 1) / QT_ROWS;
  const int lrow = tid >> 4;
  const int lchunk = tid & 15;

  for (int qt = k0 / QT_ROWS; qt < n_qt; ++qt) {
    const int q0 = qt * QT_ROWS;
    uint4 xq[4], xg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = q0 + 4 * lrow + i;
      if (r < T) {
        xq[i] = ld16(q + base + static_cast<size_t>(r) * rs + 8 * lchunk);
        xg[i] = ld16(dout + base + static_cast<size_t>(r) * rs + 8 * lchunk);
      } else {
        xq[i] = make_uint4(0, 0, 0, 0);
        xg[i] = xq[i];
      }
    }
    float l2 = 0.f, dl = 0.f;
    if (tid < QT_ROWS) {
      const int r = q0 + tid;
      l2 = r < T ? lse_bh[r] * kLog2e : INFINITY;  // padded rows get P = 0
      dl = r < T ? del_bh[r] : 0.f;
    }
    __syncthreads();
    store_tile_both(Qs, Qt, xq, lrow, lchunk);
    store_tile_both(Gs, Gt, xg, lrow, lchunk);
    if (tid < QT_ROWS) {
      lse2s[tid] = l2;
      dls[tid] = dl;
    }
    __syncthreads();

    if (q0 + QT_ROWS - 1 < kw0) continue;  // every query precedes this wavefront's keys

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc[qb] = f32x16{};
      pacc[qb] = f32x16{};
      const u16* qp = &Qs[(qb * 32 + perm_row(l32)) * RS + 8 * half];
      const u16* gp = &Gs[(qb * 32 + perm_row(l32)) * RS + 8 * half];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sacc[qb] = mfma32(as_bf16x8(ld16(qp + 16 * kc)), kreg[kc], sacc[qb]);
        pacc[qb] = mfma32(as_bf16x8(ld16(gp + 16 * kc)), vreg[kc], pacc[qb]);
      }
    }

    // lane holds key krow; element r of block qb is query q0 + 32 qb + acc_row(lane, r)
    const bool diag = q0 < kw0 + 31;
    bf16x8 pb[4], sb[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qb + acc_row(lane, r);
        float p = fast_exp2(fmaf(sacc[qb][r], c_log2, -lse2s[qi]));
        if (diag && krow > q0 + qi) p = 0.f;
        const float ds = p * (pacc[qb][r] - dls[qi]);
        pb[2 * qb + (r >> 3)][r & 7] = to_bf16(p);
        sb[2 * qb + (r >> 3)][r & 7] = to_bf16(ds);
      }

    // dV += P^T dout, dK += dS^T Q  (chunk c = queries 16 c + 8 half + 0..7)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int t = toff(db * 32 + l32, 2 * c + half);
        dva[db] = mfma32(pb[c], as_bf16x8(ld16(&Gt[t])), dva[db]);
        dka[db] = mfma32(sb[c], as_bf16x8(ld16(&Qt[t])), dka[db]);
      }
    }
  }

  // dka[db], dva[db] element r: key kw0 + 8 (r/4) + 4 half + r%4, d = 32 db + l32
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key < T) {
        const size_t off = base + static_cast<size_t>(key) * rs + 32 * db + l32;
        dk[off] = __builtin_bit_cast(u16, to_bf16(dka[db][r] * scale));
        dv[off] = __builtin_bit_cast(u16, to_bf16(dva[db][r]));
      }
    }
}

// ---------------------------------------------------------------- dQ

constexpr int DQ_ROWS = 128;  // queries per workgroup (32 per wavefront)
constexpr int DQ_KEYS = 64;   // keys per LDS tile

__global__ __launch_bounds__(256, 1) void dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    u16* __restrict__ dq, int B, int T, int H, float c_log2, float scale) {
  __shared__ __attribute__((aligned(16))) u16 Ks[DQ_KEYS * RS];
  __shared__ __attribute__((aligned(16))) u16 Vs[DQ_KEYS * RS];
  __shared__ __attribute__((aligned(16))) u16 Kt[D * DQ_KEYS];  // transposed, swizzled

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int BH = B * H;
  const int n_qt = (T + DQ_ROWS - 1) / DQ_ROWS;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.x) / BH;  // heaviest first
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / H, h = bh % H;
  const int q0 = qt * DQ_ROWS;
  const int qw0 = q0 + 32 * wave;
  const size_t rs = static_cast<size_t>(H) * D;
  const size_t base = static_cast<size_t>(b) * T * rs + static_cast<size_t>(h) * D;

  const int qrow = qw0 + l32;
  bf16x8 qreg[8], greg[8];
  float lse2 = INFINITY, dl = 0.f;
  if (qrow < T) {
    const u16* qp = q + base + static_cast<size_t>(qrow) * rs + 8 * half;
    const u16* gp = dout + base + static_cast<size_t>(qrow) * rs + 8 * half;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      qreg[kc] = as_bf16x8(ld16(qp + 16 * kc));
      greg[kc] = as_bf16x8(ld16(gp + 16 * kc));
    }
    lse2 = lse[static_cast<size_t>(bh) * T + qrow] * kLog2e;
    dl = delta[static_cast<size_t>(bh) * T + qrow];
  } else {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      qreg[kc] = as_bf16x8(make_uint4(0, 0, 0, 0));
      greg[kc] = qreg[kc];
    }
  }

  f32x16 dqa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dqa[i] = f32x16{};

  const int last_q = min(q0 + DQ_ROWS, T) - 1;
  const int n_kt = last_q / DQ_KEYS + 1;
  const int lrow = tid >> 4;
  const int lchunk = tid & 15;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * DQ_KEYS;
    uint4 xk[4], xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = k0 + 4 * lrow + i;
      if (r < T) {
        xk[i] = ld16(k + base + static_cast<size_t>(r) * rs + 8 * lchunk);
        xv[i] = ld16(v + base + static_cast<size_t>(r) * rs + 8 * lchunk);
      } else {
        xk[i] = make_uint4(0, 0, 0, 0);
        xv[i] = xk[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&Ks[(4 * lrow + i) * RS + 8 * lchunk], xk[i]);
      st16(&Vs[(4 * lrow + i) * RS + 8 * lchunk], xv[i]);
    }
    tstore_4x8(Kt, xk, lrow, lchunk);
    __syncthreads();

    if (k0 > qw0 + 31) continue;

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      pacc[kb] = f32x16{};
      const u16* kp = &Ks[(kb * 32 + perm_row(l32)) * RS + 8 * half];
      const u16* vp = &Vs[(kb * 32 + perm_row(l32)) * RS + 8 * half];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sacc[kb] = mfma32(as_bf16x8(ld16(kp + 16 * kc)), qreg[kc], sacc[kb]);
        pacc[kb] = mfma32(as_bf16x8(ld16(vp + 16 * kc)), greg[kc], pacc[kb]);
      }
    }

    const bool diag = k0 + DQ_KEYS - 1 > qw0;
    bf16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + acc_row(lane, r);
        float p = fast_exp2(fmaf(sacc[kb][r], c_log2, -lse2));
        if (diag && key > qrow) p = 0.f;
        sb[2 * kb + (r >> 3)][r & 7] = to_bf16(p * (pacc[kb][r] - dl));
      }

    // dQ^T += K^T dS^T  (chunk c = keys 16 c + 8 half + 0..7)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = as_bf16x8(ld16(&Kt[toff(db * 32 + l32, 2 * c + half)]));
        dqa[db] = mfma32(a, sb[c], dqa[db]);
      }
  }

  if (qrow < T) {
    u16* qp = dq + base + static_cast<size_t>(qrow) * rs;
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

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* delta, int B, int T, int H, hipStream_t s,
                           hipEvent_t const* ev) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float c_log2 = scale * kLog2e;
  const u16* q16 = static_cast<const u16*>(q);
  const u16* k16 = static_cast<const u16*>(k);
  const u16* v16 = static_cast<const u16*>(v);
  const u16* g16 = static_cast<const u16*>(dout);
  const long rows = static_cast<long>(B) * T * H;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  e = launch(delta_kernel, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0,
                        s, static_cast<const u16*>(o), g16, delta, B, T, H);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  const int n_kt = (T + KT_KEYS - 1) / KT_KEYS;
  e = launch(dkdv_kernel, dim3(static_cast<unsigned>(n_kt) * B * H), dim3(256), 0, s, q16, k16,
             v16, g16, lse, static_cast<const float*>(delta), static_cast<u16*>(dk),
             static_cast<u16*>(dv), B, T, H, c_log2, scale);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 2, s)) != hipSuccess) return e;
  const int n_qt = (T + DQ_ROWS - 1) / DQ_ROWS;
  e = launch(dq_kernel, dim3(static_cast<unsigned>(n_qt) * B * H), dim3(256), 0, s, q16, k16, v16,
             g16, lse, static_cast<const float*>(delta), static_cast<u16*>(dq), B, T, H, c_log2,
             scale);
  if (e != hipSuccess) return e;
  return mark(ev, 3, s);
}

}  // namespace na
