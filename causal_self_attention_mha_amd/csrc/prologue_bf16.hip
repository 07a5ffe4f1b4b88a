// Attention prologue on gfx950: QK normalisation and rotary position embedding
// of the query and key heads, forward and backward, bf16 in and out, fp32
// arithmetic.
//
// The nanochat model normalises its query and key heads and rotates them by
// position before attention (apidog blog "ChatGPTを50ドルで独自にトレーニングする
// 方法", section 1 "GPT model", architecture features).  Readings (the blog gives
// no formula): RMS normalisation over the D = 128 elements of a head with no
// learned scale, z = x / sqrt(mean(x^2) + eps); rotation of the dimension pairs
// (i, i + 64) by +theta_{p,i}, y_i = z_i cos - z_{i+64} sin,
// y_{i+64} = z_i sin + z_{i+64} cos, with cos and sin read from fp32 (T_tab, 64)
// tables at position p = t + offset[b].
//
// The work is HBM-bound (256 B read and 256 B written per head row, 12 B of
// table per element pair read from L2).  Mapping: 16 lanes own one (b, t)
// position and walk its H query rows then its H_kv key rows, lane l holding
// elements 8l .. 8l + 7 of each; the pair partner of element i < 64 sits in
// lane l + 8, one DPP row rotation away, and the RMS is a 16-lane DPP sum.  The
// lane's eight cos/sin values are loaded once per position and reused over all
// its heads; eight rows are loaded ahead of their arithmetic, and the results
// are stored non-temporally.
//
// Backward: dz = R^T dy (the rotation's transpose), then
// dx = r (dz - z mean(dz z)) with r = 1 / sqrt(mean(x^2) + eps), recomputed
// from x.
#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

// The rows are read once: non-temporal loads (d20: QK norm + RoPE forward
// 121.6 -> 118.7 us, backward 182.3 -> 172.3 us, value gate 89.4 -> 84.7 us
// forward and 89.3 -> 83.1 us backward).
#ifndef NA_PROLOGUE_NT_LOADS
#define NA_PROLOGUE_NT_LOADS 1
#endif
__device__ __forceinline__ uint4 ld_in(const void* p) {
#if NA_PROLOGUE_NT_LOADS
  return ld16_nt(p);
#else
  return ld16(p);
#endif
}

constexpr int kPosPerWg = 16;  // 4 positions per wavefront, 4 wavefronts
constexpr int kRowsAhead = 8;

// Value of x in the lane 8 apart within the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float pair_lane(float x) { return dpp<0x128>(x); }

// Sixteen-byte store that streams past the caches: the outputs are not read
// again by this kernel (measured 4% faster than a plain store at d20).
__device__ __forceinline__ void st16_stream(u16* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// BWD = false: x -> y.  BWD = true: (x, dy) -> dx.  Rows r < H come from the
// query tensors, rows H .. H + Hk - 1 from the key tensors; with xq == nullptr
// only the key rows are processed (the training forward then normalises and
// rotates the query rows itself, as it loads them).
template <bool BWD>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    const u16* __restrict__ xq, const u16* __restrict__ xk, const u16* __restrict__ gq,
    const u16* __restrict__ gk, u16* __restrict__ oq, u16* __restrict__ ok,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, const int* __restrict__ off,
    int B, int T, int H, int Hk, int T_tab, float eps) {
  const int lane = threadIdx.x & 15;
  const int pos = blockIdx.x * kPosPerWg + (threadIdx.x >> 4);
  if (pos >= B * T) return;  // no barriers below
  const int b = pos / T, t = pos - b * T;
  const int p = t + (off != nullptr ? min(max(off[b], 0), T_tab - T) : 0);

  // cos and sin for this lane's elements; the first half's partner term is
  // subtracted in the forward, so its sine is stored negated.
  const int c0 = p * 64 + (lane & 7) * 8;
  const float4 ca = *reinterpret_cast<const float4*>(cos_t + c0);
  const float4 cb = *reinterpret_cast<const float4*>(cos_t + c0 + 4);
  const float4 sa = *reinterpret_cast<const float4*>(sin_t + c0);
  const float4 sb = *reinterpret_cast<const float4*>(sin_t + c0 + 4);
  const float c[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
  const float sg = lane < 8 ? -1.f : 1.f;
  const float s[8] = {sg * sa.x, sg * sa.y, sg * sa.z, sg * sa.w,
                      sg * sb.x, sg * sb.y, sg * sb.z, sg * sb.w};

  const int R = H + Hk;
  // element offset of this lane's slice of row r in its (B, T, H or Hk, D) tensor
  auto row = [&](int r) -> size_t {
    return r < H ? ((size_t)pos * H + r) * kHeadDim + lane * 8
                 : ((size_t)pos * Hk + (r - H)) * kHeadDim + lane * 8;
  };
  for (int r0 = xq != nullptr ? 0 : H; r0 < R; r0 += kRowsAhead) {
    uint4 xv[kRowsAhead], gv[kRowsAhead];
#pragma unroll
    for (int u = 0; u < kRowsAhead; ++u) {
      const int r = r0 + u;
      if (r < R) {
        const size_t o = row(r);
        xv[u] = ld_in((r < H ? xq : xk) + o);
        if (BWD) gv[u] = ld_in((r < H ? gq : gk) + o);
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsAhead; ++u) {
      const int r = r0 + u;
      if (r >= R) break;
      float x[8], y[8];
      unpack8(xv[u], x);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
      const float rs = __builtin_amdgcn_rsqf(sum16(ss) * (1.f / kHeadDim) + eps);
      if (!BWD) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float z = x[i] * rs;
          y[i] = fmaf(z, c[i], s[i] * pair_lane(z));
        }
      } else {
        float g[8], dz[8];
        unpack8(gv[u], g);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dz[i] = fmaf(g[i], c[i], -s[i] * pair_lane(g[i]));
          dot = fmaf(dz[i], x[i], dot);
        }
        // mean(dz z) = rs * sum(dz x) / D
        const float m = sum16(dot) * rs * (1.f / kHeadDim);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = rs * fmaf(-x[i] * rs, m, dz[i]);
      }
      st16_stream((r < H ? oq : ok) + row(r), pack8(y));
    }
  }
}

// Value-embedding gate (ResFormer value residual, same blog and section):
// v' = v + 3 sigmoid(g) ve per key/value head row, g (B, T, Hk) the gate
// logits.  Backward: dv = dv' (the caller reuses it, nothing is written),
// dve = 3 sigmoid(g) dv', dg = 3 sigmoid(g) (1 - sigmoid(g)) <ve, dv'>.
// 16 lanes per row as above, kRowsAhead consecutive rows per 16-lane group.
template <bool BWD>
__global__ __launch_bounds__(256) void value_gate_kernel(const u16* __restrict__ a,
                                                         const u16* __restrict__ ve,
                                                         const u16* __restrict__ gate,
                                                         u16* __restrict__ out,
                                                         u16* __restrict__ dgate, long rows) {
  const int lane = threadIdx.x & 15;
  const long r0 = ((long)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4)) * kRowsAhead;
  uint4 av[kRowsAhead], ev[kRowsAhead];
  float gv[kRowsAhead];
#pragma unroll
  for (int u = 0; u < kRowsAhead; ++u)
    if (r0 + u < rows) {
      const size_t o = (size_t)(r0 + u) * kHeadDim + lane * 8;
      av[u] = ld_in(a + o);
      ev[u] = ld_in(ve + o);
      gv[u] = bf16_to_f32(gate[r0 + u]);
    }
#pragma unroll
  for (int u = 0; u < kRowsAhead; ++u) {
    if (r0 + u >= rows) break;
    const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-gv[u] * 1.4426950408889634f));
    float x[8], e[8], y[8];
    unpack8(av[u], x);
    unpack8(ev[u], e);
    if (!BWD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fmaf(3.f * sg, e[i], x[i]);
    } else {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y[i] = 3.f * sg * x[i];
        dot = fmaf(e[i], x[i], dot);
      }
      dot = sum16(dot);
      if (lane == 0) dgate[r0 + u] = __builtin_bit_cast(u16, to_bf16(3.f * sg * (1.f - sg) * dot));
    }
    st16_stream(out + (size_t)(r0 + u) * kHeadDim + lane * 8, pack8(y));
  }
}

}  // namespace

hipError_t launch_value_gate_bf16(const void* a, const void* ve, const void* gate, void* out,
                                  void* dgate, int B, int T, int Hk, bool backward,
                                  hipStream_t s) {
  const long rows = (long)B * T * Hk;
  const long per_wg = 16 * kRowsAhead;
  const dim3 grid((unsigned)((rows + per_wg - 1) / per_wg)), block(256);
  auto ca = static_cast<const u16*>(a), cv = static_cast<const u16*>(ve),
       cg = static_cast<const u16*>(gate);
  if (backward)
    return launch(value_gate_kernel<true>, grid, block, 0, s, ca, cv, cg, static_cast<u16*>(out),
                  static_cast<u16*>(dgate), rows);
  return launch(value_gate_kernel<false>, grid, block, 0, s, ca, cv, cg, static_cast<u16*>(out),
                static_cast<u16*>(nullptr), rows);
}

hipError_t launch_qk_norm_rope_bf16(const void* q, const void* k, const void* dyq,
                                    const void* dyk, void* outq, void* outk, const float* cos_t,
                                    const float* sin_t, const int* off, int B, int T, int H,
                                    int Hk, int T_tab, float eps, bool backward, hipStream_t s) {
  const int n_pos = B * T;
  const dim3 grid((n_pos + kPosPerWg - 1) / kPosPerWg), block(256);
  auto cq = static_cast<const u16*>(q), ck = static_cast<const u16*>(k);
  auto oq = static_cast<u16*>(outq), ok = static_cast<u16*>(outk);
  if (backward)
    return launch(qk_norm_rope_kernel<true>, grid, block, 0, s, cq, ck,
                  static_cast<const u16*>(dyq), static_cast<const u16*>(dyk), oq, ok, cos_t, sin_t,
                  off, B, T, H, Hk, T_tab, eps);
  return launch(qk_norm_rope_kernel<false>, grid, block, 0, s, cq, ck,
                static_cast<const u16*>(nullptr), static_cast<const u16*>(nullptr), oq, ok, cos_t,
                sin_t, off, B, T, H, Hk, T_tab, eps);
}

}  // namespace na
