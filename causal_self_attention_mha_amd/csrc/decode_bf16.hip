// bf16 single-token decode over a ragged, padded KV cache (split-KV).
//
// Per (b, h), with L = seqlens[b] clamped to [0, T_cap]:
//   z_j = s <q_bh, K[b, j, h]>  (j < L),  o = softmax(z) V[b, 0:L, h],
//   lse = ln sum_j exp(z_j)
// i.e. the attention step nanochat's inference engine runs per generated
// token against its prefilled prompt cache through flash_attn_with_kvcache
// (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法", section 6
// "inference engine"); the new token's key and value are already in the cache
// at row L-1.
//
// The work is HBM bound (each cached K and V byte is used once).  Two kernels:
//   split:   one workgroup per (chunk of 256 keys, b) holding keys < L, all
//            heads together.  16-lane groups map to (head h, stream s); at a
//            given loop step the groups of all heads and streams read whole
//            cache rows (S * H * 256 contiguous bytes of K and of V), so the
//            cache streams from HBM in order.  One pass: each group takes its
//            keys in batches of 8, with the next batch's K and V loads in
//            flight while the current batch runs an online softmax (running
//            max, sum and output in registers); no barrier until the streams
//            of a head are merged through LDS at the end.  Writes unnormalised
//            o_c and (m_c, l_c) per (b, chunk, h).
//   combine: one workgroup per (b, h): o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Rows t >= L are never read.
#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr int CHUNK = 256;  // keys per split workgroup
constexpr int U = 8;        // keys per batch and per lane

__host__ __device__ inline int n_chunks(int T_cap) { return (T_cap + CHUNK - 1) / CHUNK; }

// Streams per head: enough 16-lane groups to reach at least 256 threads, at
// most 512 threads (H <= 32 is checked on the host).
inline int streams_for(int H) {
  const int s = (256 + 16 * H - 1) / (16 * H);
  return s * 16 * H <= 512 ? s : 1;
}

// workspace: o_part [B][NC][H][D] fp32, then ml [B][NC][H][2] fp32 (m_c, l_c)
__global__ __launch_bounds__(512) void decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int* __restrict__ seqlens, float* __restrict__ opart, float* __restrict__ ml, int H,
    int T_cap, int S, float scale) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* part = smem;                    // [S][H][D] per-stream outputs
  float* pm = part + S * H * D;          // [S][H] per-stream running max
  float* pl = pm + S * H;                // [S][H] per-stream running sum

  const int c = blockIdx.x, b = blockIdx.y;
  const int NC = gridDim.x;
  const int L = min(max(seqlens[b], 0), T_cap);
  const int j0 = c * CHUNK;
  if (j0 >= L) return;  // uniform across the workgroup
  const int n = min(CHUNK, L - j0);

  const int tid = threadIdx.x;
  const int g = tid >> 4;       // group
  const int l16 = tid & 15;     // which 16 bytes of the 256-byte head row
  const int h = g % H;
  const int st = g / H;         // stream
  const size_t rs = static_cast<size_t>(H) * D;
  const size_t base = (static_cast<size_t>(b) * T_cap + j0) * rs + static_cast<size_t>(h) * D +
                      8 * l16;
  const u16* kb = kc + base;
  const u16* vb = vc + base;

  float qv[8];  // q scaled by s * log2(e): scores come out in the exp2 domain
  {
    const float c2 = scale * 1.4426950408889634f;
    const uint4 x = ld16(q + (static_cast<size_t>(b) * H + h) * D + 8 * l16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u = (&x.x)[w];
      qv[2 * w] = __uint_as_float(u << 16) * c2;
      qv[2 * w + 1] = __uint_as_float(u & 0xffff0000u) * c2;
    }
  }

  // keys st, st + S, ... (< n) in batches of U; rows past n re-read row n-1
  // and get zero weight
  auto row = [&](int key) { return static_cast<size_t>(min(key, n - 1)) * rs; };
  uint4 xk[U], xv[U], yk[U], yv[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    xk[i] = ld16(kb + row(st + i * S));
    xv[i] = ld16(vb + row(st + i * S));
  }
  float m = -INFINITY, l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = st; k0 < n; k0 += U * S) {
    const int k1 = k0 + U * S;  // next batch (clamped loads are harmless past n)
#pragma unroll
    for (int i = 0; i < U; ++i) {
      yk[i] = ld16(kb + row(k1 + i * S));
      yv[i] = ld16(vb + row(k1 + i * S));
    }
    float z[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = (&xk[i].x)[w];
        a = fmaf(qv[2 * w], __uint_as_float(u << 16), a);
        a = fmaf(qv[2 * w + 1], __uint_as_float(u & 0xffff0000u), a);
      }
      a = sum16(a);
      z[i] = k0 + i * S < n ? a : -INFINITY;
    }
    float bm = z[0];
#pragma unroll
    for (int i = 1; i < U; ++i) bm = fmaxf(bm, z[i]);
    const float m_new = fmaxf(m, bm);        // finite: key k0 < n is valid
    const float alpha = fast_exp2(m - m_new);  // 0 on the first batch
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const float p = fast_exp2(z[i] - m_new);  // 0 for dropped rows
      l += p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = (&xv[i].x)[w];
        acc[2 * w] = fmaf(p, __uint_as_float(u << 16), acc[2 * w]);
        acc[2 * w + 1] = fmaf(p, __uint_as_float(u & 0xffff0000u), acc[2 * w + 1]);
      }
    }
    m = m_new;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      xk[i] = yk[i];
      xv[i] = yv[i];
    }
  }

  // merge the S streams of each head (in the exp2 domain), stream 0 writes
  float* pp = part + (static_cast<size_t>(st) * H + h) * D + 8 * l16;
#pragma unroll
  for (int e = 0; e < 8; ++e) pp[e] = acc[e];
  if (l16 == 0) {
    pm[st * H + h] = m;  // -inf for a stream that had no key
    pl[st * H + h] = l;
  }
  __syncthreads();
  if (st == 0) {
    float M = -INFINITY;
    for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, pm[s2 * H + h]);
    float out[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int s2 = 0; s2 < S; ++s2) {
      const float w = fast_exp2(pm[s2 * H + h] - M);
      den = fmaf(w, pl[s2 * H + h], den);
      const float* sp = part + (static_cast<size_t>(s2) * H + h) * D + 8 * l16;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = fmaf(w, sp[e], out[e]);
    }
    const size_t slot = (static_cast<size_t>(b) * NC + c) * H + h;
    float* op = opart + slot * D + 8 * l16;
    *reinterpret_cast<float4*>(op) = make_float4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<float4*>(op + 4) = make_float4(out[4], out[5], out[6], out[7]);
    if (l16 == 0) {
      ml[2 * slot] = M * 0.6931471805599453f;  // back to natural-log units
      ml[2 * slot + 1] = den;
    }
  }
}

__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ ml,
    const int* __restrict__ seqlens, u16* __restrict__ o, float* __restrict__ lse, int H,
    int T_cap, int NC) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), T_cap);
  const int nc = (L + CHUNK - 1) / CHUNK;
  const int d = threadIdx.x;
  const float* mlb = ml + 2 * (static_cast<size_t>(b) * NC * H + h);  // chunk c at 2 c H
  const float* opb = opart + (static_cast<size_t>(b) * NC * H + h) * D + d;  // chunk c at c H D
  // groups of 16 chunks: all loads of a group issued before they are used
  constexpr int G = 16;
  float M = -INFINITY;
  for (int c0 = 0; c0 < nc; c0 += G) {
    float mv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) mv[i] = c0 + i < nc ? mlb[2 * (c0 + i) * H] : -INFINITY;
#pragma unroll
    for (int i = 0; i < G; ++i) M = fmaxf(M, mv[i]);
  }
  float den = 0.f, num = 0.f;
  for (int c0 = 0; c0 < nc; c0 += G) {
    float mv[G], lv[G], ov[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool ok = c0 + i < nc;
      const int c = ok ? c0 + i : c0;
      mv[i] = ok ? mlb[2 * c * H] : -INFINITY;
      lv[i] = mlb[2 * c * H + 1];
      ov[i] = opb[static_cast<size_t>(c) * H * D];
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float w = expf(mv[i] - M);  // 0 for chunks past nc
      den = fmaf(w, lv[i], den);
      num = fmaf(w, ov[i], num);
    }
  }
  const float out = nc > 0 ? num / den : 0.f;
  o[(static_cast<size_t>(b) * H + h) * D + d] = __builtin_bit_cast(u16, to_bf16(out));
  if (lse != nullptr && d == 0)
    lse[static_cast<size_t>(b) * H + h] = nc > 0 ? M + logf(den) : -INFINITY;
}

}  // namespace

std::size_t decode_workspace_bytes(int B, int H, int T_cap) {
  const std::size_t slots = static_cast<std::size_t>(B) * n_chunks(T_cap) * H;
  return slots * (D + 2) * sizeof(float);
}

hipError_t launch_decode_bf16(const void* q, const void* kc, const void* vc, const int* seqlens,
                              void* o, float* lse, int B, int H, int T_cap, void* ws,
                              hipStream_t s, hipEvent_t const* ev) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int NC = n_chunks(T_cap);
  const int S = streams_for(H);
  const int threads = 16 * H * S;
  const size_t shmem = (static_cast<size_t>(S) * H * D + 2 * static_cast<size_t>(S) * H) *
                       sizeof(float);
  float* opart = static_cast<float*>(ws);
  float* ml = opart + static_cast<std::size_t>(B) * NC * H * D;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  e = launch(decode_split_kernel, dim3(NC, B), dim3(threads), shmem, s, static_cast<const u16*>(q),
             static_cast<const u16*>(kc), static_cast<const u16*>(vc), seqlens, opart, ml, H,
             T_cap, S, scale);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  e = launch(decode_combine_kernel, dim3(H, B), dim3(128), 0, s, static_cast<const float*>(opart),
             static_cast<const float*>(ml), seqlens, static_cast<u16*>(o), lse, H, T_cap, NC);
  if (e != hipSuccess) return e;
  return mark(ev, 2, s);
}

}  // namespace na
