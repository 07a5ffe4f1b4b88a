// bf16 causal attention forward on gfx950 MFMA.
//
// Computes, per (batch b, head h), o = softmax(s q k^T + causal mask) v and
// lse = ln(row sums), the attention nanochat runs through
// flash_attn_func(q, k, v, causal=True) (apidog blog "ChatGPTを50ドルで独自に
// トレーニングする方法", section 5 "Flash Attention integration"), with
// s = 1/sqrt(128) and key j visible to query i iff j <= i.
//
// Design (one workgroup = 4 wavefronts = 128 query rows of one (b, h)):
//   * each wavefront owns 32 query rows; its Q^T operand (32 x 128 bf16) stays
//     in registers for the whole key loop;
//   * K and V tiles of 64 keys are copied straight from HBM into
//     double-buffered LDS (buffer loads with the LDS destination; keys past T
//     arrive as zeros), the next tile's copy issued after the current tile's
//     score MFMAs and in flight during its softmax and PV; one barrier per
//     tile.  Both tiles keep their natural row-major layout, swizzled (see
//     tile_swz): K is read row-wise, V^T with the transposing
//     ds_read_b64_tr_b16, both free of bank conflicts;
//   * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//     so that each lane owns one query row: the online-softmax max and sum are
//     lane-local apart from one exchange with lane l^32;
//   * the output is accumulated transposed too, O^T += V^T P^T, so the per-row
//     rescale factor is also lane-local;
//   * the softmax runs in the exp2 domain: p = 2^(c z - c m) with c =
//     s log2(e).  In the training forward (no window, no prefill) Q is
//     pre-scaled by c and rounded to bf16 (as the dK/dV pass does with K) and
//     the score chains start from -m (the MFMA's accumulator input), so a
//     score costs one v_exp_f32 and nothing else: m is set by a wavefront's
//     first tile and raised only when a lane's probability sum over a tile
//     reaches 2^31; the other instantiations take one FMA per score against
//     a running max raised lazily;
//   * the 32 LDS operand reads of a tile are issued in a fixed order four
//     operands ahead of the MFMA that consumes them, the last K MFMAs
//     overlapping the first V reads, which in turn stay in flight during the
//     softmax;
//   * key tiles entirely above the diagonal are never visited; only tiles that
//     cross the diagonal apply the causal select;
//   * each XCD runs a group of heads' query tiles together, heaviest first
//     (the query heads that share a key/value head next to each other), so
//     their K and V stay in that XCD's L2.
// The same kernel, instantiated with WIN and PRE, serves sliding windows and
// the prefill of a chunk over a KV cache (see the template's notes).
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int D = kHeadDim;
#ifndef NA_FWD_NW
#define NA_FWD_NW 4
#endif
constexpr int NW = NA_FWD_NW;     // wavefronts per workgroup (32 query rows each)
constexpr int BQ = 32 * NW;       // query rows per workgroup
constexpr int BK = 64;   // keys per LDS tile
constexpr uint32_t BUF_B = 2 * kTileBytes;  // one buffer: K tile, then V tile
// Lazy rescaling: the running max m is only raised (and O, l rescaled) when a
// new score exceeds it by more than 2^8 in the exp2 domain, so most tiles skip
// the rescale; probabilities then stay below 256, harmless in fp32 and bf16.
constexpr float kRescaleLog2 = 8.0f;
// The training forward's offset m is raised only when a lane's probability
// sum over one tile reaches this (every probability then stays below it).
constexpr float kSumLimit = 2147483648.0f;  // 2^31

// WIN: sliding window, key j visible to query i iff i - win <= j <= i (the
// plain causal kernel is WIN = false).
// PRE: prefill over a KV cache.  q, o hold T query rows per sequence, k, v are
// caches of Tc rows per sequence, and the query rows sit at positions
// L .. L + T - 1 with L = lens[b] (clamped to [0, Tc - T]): query row r sees
// cache rows 0 .. L + r.  Without PRE, Tc = T and L = 0 (training).  Masks and
// tile ranges below compare key rows with query positions L + r.
// ROPE: q holds the raw query heads; each row is RMS-normalised and rotated by
// the angles of its position (fp32 (T_tab, 64) cos/sin tables) as it is
// loaded, then rounded to bf16 like any query operand.  In the training
// forward (no PRE) the rotated bf16 rows are also written to qo, the query
// operand of the backward.
template <bool WIN, bool PRE, bool ROPE = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ o, float* __restrict__ lse, int B, int T, int Tc, int H, int Hk,
    const int* __restrict__ lens, float c_log2, float scale, int win,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, float eps,
    u16* __restrict__ qo) {
  // two buffers of (K tile, V tile), swizzled (see tile_swz)
  __shared__ __attribute__((aligned(1024))) char kvs[2 * BUF_B];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;   // which 8-wide k half of an MFMA operand
  const int l32 = lane & 31;

  const int n_qt = (T + BQ - 1) / BQ;
  // Items are grouped by key/value head: the G = H / Hk query heads that read
  // one K, V head run on one XCD next to each other (query head fastest), so
  // its K and V stay in that XCD's L2.
  const int G = H / Hk;
  int bhk, tg;
  xcd_tile_map_grouped(static_cast<int>(blockIdx.x), B * Hk, n_qt * G, kHeadGroup, bhk, tg);
  const int qt = n_qt - 1 - tg / G;  // heaviest (last) query tile first
  const int b = bhk / Hk, hk = bhk % Hk;
  const int h = hk * G + tg % G;
  const int bh = b * H + h;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;
  const int L = PRE ? min(max(lens[b], 0), Tc - T) : 0;  // position of query row 0
  const int nk = PRE ? L + T : T;                          // key rows that exist
  // 32-bit row offsets within one batch (T * H * D < 2^31 is checked on the host)
  const int rs = H * D;    // q, o: stride between t
  const int rsk = Hk * D;  // k, v
  const size_t base = static_cast<size_t>(b) * T * rs + static_cast<size_t>(h) * D;
  const size_t kbase =
      static_cast<size_t>(b) * (PRE ? Tc : T) * rsk + static_cast<size_t>(hk) * D;

  const int last_q = L + min(q0 + BQ, T) - 1;  // position of the last query row
  const int n_kt = last_q / BK + 1;  // key tiles at or left of the diagonal
  // first key tile that any row of the workgroup sees (0 without a window)
  const int kt_lo = WIN ? max(L + q0 - win, 0) / BK : 0;
  const uint32_t kv_lds = lds_addr(kvs);
  const uint32_t rsb = static_cast<uint32_t>(rsk) * 2;
  const uint32_t cvoff = tile_copy_offset(wave, lane, rsb);
  auto issue = [&](int kt, int buf) {  // K, V tile kt -> buffer buf; keys past nk read as 0
    const int k0 = kt * BK;
    const uint32_t nrec = static_cast<uint32_t>(nk - k0) * rsb;
    const size_t off = kbase + static_cast<size_t>(k0) * rsk;
    copy_tile<NW>(buffer_rsrc(k + off, nrec), cvoff, rsb, kv_lds + buf * BUF_B, wave);
    copy_tile<NW>(buffer_rsrc(v + off, nrec), cvoff, rsb, kv_lds + buf * BUF_B + kTileBytes,
                  wave);
  };
  // the first K/V tile's copy goes out before the Q loads, whose use (the
  // pre-scale, the prologue) would otherwise hold it back
  issue(kt_lo, 0);

  // Q^T operand: lane holds q[qw0 + l32][16 kc + 8 half + 0..7], kc = 0..7.
  // Rows past T (their outputs are discarded) read row T-1 instead.
  const int qrow = qw0 + l32;
  // the training forward: Q pre-scaled, score chains seeded with -m (see above)
  constexpr bool DIET = !WIN && !PRE;
  bf16x8 qreg[8];
  {
    const u16* qp = q + base + min(qrow, T - 1) * rs + 8 * half;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qreg[kc] = as_bf16x8(ld16(qp + 16 * kc));
  }
  if constexpr (ROPE) {
    // the lane holds elements 16 kc + 8 half + e of its row; element i < 64
    // (kc < 4) pairs with i + 64, the same e of qreg[kc + 4]; the other half
    // of the row sits in lane l ^ 32
    // the angles are loaded first, so that they are in flight with the rows
    const int p = L + min(qrow, T - 1);  // the row's position in the cache
    const float* cp = cos_t + static_cast<size_t>(p) * (D / 2) + 8 * half;
    const float* sp = sin_t + static_cast<size_t>(p) * (D / 2) + 8 * half;
    float4 ang[4][4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      ang[kc][0] = *reinterpret_cast<const float4*>(cp + 16 * kc);
      ang[kc][1] = *reinterpret_cast<const float4*>(cp + 16 * kc + 4);
      ang[kc][2] = *reinterpret_cast<const float4*>(sp + 16 * kc);
      ang[kc][3] = *reinterpret_cast<const float4*>(sp + 16 * kc + 4);
    }
    float x[8][8];
    float ss = 0.f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[kc][e] = static_cast<float>(qreg[kc][e]);
        ss = fmaf(x[kc][e], x[kc][e], ss);
      }
    ss += __shfl_xor(ss, 32, 64);
    const float r = __builtin_amdgcn_rsqf(ss * (1.f / D) + eps);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const float4 c0 = ang[kc][0], c1 = ang[kc][1], s0 = ang[kc][2], s1 = ang[kc][3];
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float z1 = x[kc][e] * r, z2 = x[kc + 4][e] * r;
        qreg[kc][e] = to_bf16(fmaf(z1, cs[e], -z2 * sn[e]));
        qreg[kc + 4][e] = to_bf16(fmaf(z1, sn[e], z2 * cs[e]));
      }
    }
    if constexpr (!PRE) {  // the rotated rows: the backward's q operand
      if (qrow < T) {
        u16* op = qo + base + static_cast<size_t>(qrow) * rs + 8 * half;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) st16(op + 16 * kc, __builtin_bit_cast(uint4, qreg[kc]));
      }
    }
  }
  if constexpr (DIET) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[kc][e] = to_bf16(static_cast<float>(qreg[kc][e]) * c_log2);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;  // running max of raw scores for row qrow (DIET: the
                        // offset of the scaled scores, set by the first tile)
  float lpart = 0.f;    // running sum over this lane's half of the keys
  const float thr = kRescaleLog2 / c_log2;
  f32x16 ofs;  // DIET: -m in every element, the score chains' initial value
#pragma unroll
  for (int e = 0; e < 16; ++e) ofs[e] = 0.f;
  bool mset = false;  // DIET: m set (wavefront-uniform: a wavefront's rows share their tiles)


  // operand read addresses in buffer 0 (buffer 1: + BUF_B, V tile: + kTileBytes)
  TileAddr ta;
  {
    const TileOffsets ofs = tile_operand_offsets(lane);
    nat_addr(kv_lds, ofs, ta.nat);
    tr_addr(kv_lds + kTileBytes, ofs, ta.tr);
  }

  // One key tile; BUF is the buffer it sits in (a compile-time constant, so
  // that every LDS read address is a register plus an immediate).
  auto tile = [&](auto bufc, int kt) {
    constexpr uint32_t BUF = decltype(bufc)::value;
    constexpr uint32_t KO = BUF * BUF_B;  // K tile offset from buffer 0's
    constexpr uint32_t VO = BUF * BUF_B;  // V^T reads: ta.tr already points at the V tile
    const int k0 = kt * BK;
    // One barrier per tile: after it every copy into this buffer has landed
    // and every wavefront is done with the other buffer (tile kt-1), which the
    // next copy may then overwrite.
    if constexpr (ROPE && !PRE) {
      // first tile: the 8 stores of the rotated query rows went out after its
      // copy (all 8 whenever the wavefront's first row is below T); vector
      // memory operations retire in issue order, so the copy has landed once
      // at most those 8 are outstanding, and the stores need not be waited for
      if (kt == kt_lo && qw0 < T)
        wait_vmem_but<8>();
      else
        wait_vmem();
    } else {
      wait_vmem();
    }
    wait_lds();
    __syncthreads();
    // whole tile above this wavefront's diagonal, or before its rows' windows
    const bool skip = k0 > L + qw0 + 31 || (WIN && k0 + BK - 1 < L + qw0 - win);
    // The copy of the next tile is issued once this tile's K reads are done
    // (measured faster than issuing it at the barrier).
    if (skip) {
      if (kt + 1 < n_kt) issue(kt + 1, 1 - BUF);
      return;
    }

    // Operand sequence: 16 K operands, n = 2 kc + kb (the two score blocks
    // alternate, so consecutive MFMAs are independent), then 16 V^T operands,
    // n = 16 + 4 c + db.
    bf16x8 opnd[32];
    auto read = [&](int n) {
      if (n < 16) {
        const int kc = n >> 1, kb = n & 1;
        opnd[n] = as_bf16x8(lds_ld16(ta.nat[kc] + KO + kb * 32 * 256));
      } else {
        const int c = (n - 16) >> 2, db = (n - 16) & 3;
        opnd[n] = tr_operand(ta.tr[db], VO + c * 16 * 256);
      }
    };
    constexpr int AHEAD = 4;
#pragma unroll
    for (int n = 0; n < AHEAD; ++n) read(n);
    __builtin_amdgcn_sched_barrier(0);

    // S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      read(n + AHEAD);
      sacc[n & 1] = mfma32(opnd[n], qreg[n >> 1], (DIET && n < 2) ? ofs : sacc[n & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < n_kt) issue(kt + 1, 1 - BUF);

    // causal select on tiles that cross the diagonal (and, with a window, on
    // tiles that cross the lower edge of some row's window)
    if (k0 + BK - 1 > L + qw0 || (WIN && k0 < L + qw0 + 31 - win)) {
      const int qpos = L + qrow;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + acc_row(lane, r);
          if (key > qpos || (WIN && key < qpos - win)) sacc[kb][r] = -INFINITY;
        }
    }

    // the largest of this lane's scores, shared with lane l ^ 32 (same row)
    auto tile_max = [&]() {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      return fmaxf(mx, __shfl_xor(mx, 32, 64));
    };
    // P^T as bf16 MFMA B operands: chunk c (16 keys) = sacc[c/2][8(c%2) .. +7]
    bf16x8 pb[4];
    float psum = 0.f;
    if constexpr (DIET) {
      // sacc holds c z - m (c z on the wavefront's first tile, which sets m)
      if (!mset) {
        m = tile_max();  // finite: every row sees key 0 in its first tile
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] -= m;
#pragma unroll
        for (int e = 0; e < 16; ++e) ofs[e] = -m;
        mset = true;
      }
      auto probs = [&](float sh) {  // p = 2^(sacc - sh)
        psum = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = fast_exp2(sacc[c >> 1][8 * (c & 1) + i] - sh);
            psum += p;
            pb[c][i] = to_bf16(p);
          }
      };
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(sacc[c >> 1][8 * (c & 1) + i]);
          psum += p;
          pb[c][i] = to_bf16(p);
        }
      if (__any(!(psum < kSumLimit))) {  // rare: scores far above m (wavefront-uniform)
        const float dm = fmaxf(tile_max(), 0.f);
        const float alpha = fast_exp2(-dm);
        lpart *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m += dm;
#pragma unroll
        for (int e = 0; e < 16; ++e) ofs[e] = -m;
        probs(dm);
      }
    } else {
      const float mx = tile_max();
      if (__any(mx > m + thr)) {  // wavefront-uniform
        const float m_new = fmaxf(m, mx);
        // 0 on the first tile; with a window, a row whose keys so far all lie
        // before its window keeps m = -inf (and l = 0, O = 0): any finite factor
        const float alpha =
            (WIN && m_new == -INFINITY) ? 0.f : fast_exp2((m - m_new) * c_log2);
        lpart *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m = m_new;
      }
      // a row whose keys so far all lie before its window (WIN only) still has
      // m = -inf: its probabilities are exp2(-inf) = 0, not exp2(-inf + inf)
      const float neg = (WIN && m == -INFINITY) ? 0.f : -m * c_log2;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(fmaf(sacc[c >> 1][8 * (c & 1) + i], c_log2, neg));
          psum += p;
          pb[c][i] = to_bf16(p);
        }
      }
    }
    lpart += psum;
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P^T
#pragma unroll
    for (int n = 16; n < 32; ++n) {
      if (n + AHEAD < 32) read(n + AHEAD);
      const int c = (n - 16) >> 2, db = (n - 16) & 3;
      oacc[db] = mfma32(opnd[n], pb[c], oacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int kt = kt_lo; kt < n_kt; kt += 2) {
    tile(std::integral_constant<uint32_t, 0>{}, kt);
    if (kt + 1 < n_kt) tile(std::integral_constant<uint32_t, 1>{}, kt + 1);
  }

  const float l = lpart + __shfl_xor(lpart, 32, 64);
  // The rows leave through this wavefront's 8 KiB of the K/V buffers (free
  // once every wavefront is past its last tile), so that 16 lanes store one
  // 256-byte row (chunk c of row r at c ^ (r % 16)); stored straight from the
  // accumulators, every lane wrote 8 bytes to a different row (d20 forward
  // 394 -> 388 us).
  wait_lds();
  __syncthreads();
  {
    const float inv = 1.f / l;
    const uint32_t stg = kv_lds + wave * 8192;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // elements 4g..4g+3 are d = 32 db + 8 g + 4 half + 0..3
        lds_st8(stg + l32 * 256 + 16 * ((4 * db + g) ^ (l32 & 15)) + 8 * half,
                pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv));
      }
    asm volatile("" ::: "memory");  // the reads below follow the writes above
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {  // lane i: chunk i % 16 of row 4 mm + i / 16
      const int rr = 4 * mm + (lane >> 4), c = lane & 15;
      const uint4 x = lds_ld16(stg + rr * 256 + 16 * (c ^ (rr & 15)));
      if (qw0 + rr < T) st16(o + base + static_cast<size_t>(qw0 + rr) * rs + 8 * c, x);
    }
  }
  if (qrow < T) {
    if (half == 0 && (!PRE || lse != nullptr))
      lse[static_cast<size_t>(bh) * T + qrow] =
          DIET ? (m + __log2f(l)) * 0.6931471805599453f : m * scale + logf(l);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int T, int H, int Hk, int window, hipStream_t s,
                           const float* cos_t, const float* sin_t, float eps, void* q_rot) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float c_log2 = scale * 1.4426950408889634f;
  const int n_qt = (T + BQ - 1) / BQ;
  const dim3 grid(static_cast<unsigned>(n_qt) * B * H);
  const bool win = window >= 0 && window < T - 1;  // else every row sees all its keys
  const bool rope = cos_t != nullptr;
  auto* kern = rope ? (win ? fwd_bf16_kernel<true, false, true> : fwd_bf16_kernel<false, false, true>)
                    : (win ? fwd_bf16_kernel<true, false> : fwd_bf16_kernel<false, false>);
  return launch(kern, grid, dim3(64 * NW), 0, s, static_cast<const u16*>(q),
                static_cast<const u16*>(k), static_cast<const u16*>(v), static_cast<u16*>(o), lse,
                B, T, T, H, Hk, static_cast<const int*>(nullptr), c_log2, scale,
                win ? window : T, cos_t, sin_t, eps, static_cast<u16*>(q_rot));
}

// Prefill: the T new rows of k_new, v_new go to cache rows L .. L + T - 1
// (L = lens[b] clamped to [0, Tc - T]), one 16-byte chunk per thread; the
// rows of one (b, t) are contiguous (H_kv D elements) in both tensors.
// ROPE: each key head row is RMS-normalised and rotated by the angles of its
// position L + t on the way (16 lanes per head row: the pair partner of
// element i < 64 is 8 lanes away, the sum of squares a 16-lane sum).
// GATE: each value head row gets the value-embedding gate on the way,
// v + 3 sigmoid(g) ve, with ve (B, T, Hk, D) and the logits g (B, T, Hk) bf16.
template <bool ROPE, bool GATE>
__global__ __launch_bounds__(256) void kv_append_kernel(const u16* __restrict__ k_new,
                                                        const u16* __restrict__ v_new,
                                                        u16* __restrict__ kc, u16* __restrict__ vc,
                                                        const int* __restrict__ lens, int T,
                                                        int Tc, int Hk, long chunks,
                                                        const float* __restrict__ cos_t,
                                                        const float* __restrict__ sin_t,
                                                        float eps, const u16* __restrict__ ve,
                                                        const u16* __restrict__ gate) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= chunks) return;  // chunks is a multiple of 16: whole head rows drop out
  const int per_row = Hk * D / 8;  // 16-byte chunks per (b, t) row
  const long row = i / per_row;    // b * T + t
  const int c = static_cast<int>(i - row * per_row);
  const int b = static_cast<int>(row / T), t = static_cast<int>(row - static_cast<long>(b) * T);
  const int L = min(max(lens[b], 0), Tc - T);
  const size_t dst = (static_cast<size_t>(b) * Tc + L + t) * Hk * D + 8 * c;
  const size_t src = static_cast<size_t>(row) * Hk * D + 8 * c;
  uint4 kv = ld16(k_new + src);
  if constexpr (ROPE) {
    const int sub = c & 15;  // elements 8 sub .. 8 sub + 7 of the head row
    const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
    float x[8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      ss = fmaf(x[2 * j], x[2 * j], fmaf(x[2 * j + 1], x[2 * j + 1], ss));
    }
    const float r = __builtin_amdgcn_rsqf(sum16(ss) * (1.f / D) + eps);
    const size_t tp = static_cast<size_t>(L + t) * (D / 2) + 8 * (sub & 7);
    const float sg = sub < 8 ? -1.f : 1.f;  // y_i = z_i c - z_{i+64} s, y_{i+64} = z_i s + z_{i+64} c
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float z = x[e] * r;
      const float zp = dpp<0x128>(z);  // the partner lane's element (row_ror:8)
      y[e] = fmaf(z, cos_t[tp + e], sg * sin_t[tp + e] * zp);
    }
    kv = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                    pack_bf16x2(y[6], y[7]));
  }
  st16(kc + dst, kv);
  uint4 vv = ld16(v_new + src);
  if constexpr (GATE) {
    const float g = bf16_to_f32(gate[row * Hk + c / 16]);
    const float w3 = 3.f * __builtin_amdgcn_rcpf(1.f + fast_exp2(-g * 1.4426950408889634f));
    const uint4 ev = ld16(ve + src);
    const uint32_t a[4] = {vv.x, vv.y, vv.z, vv.w}, b4[4] = {ev.x, ev.y, ev.z, ev.w};
    uint32_t r4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r4[j] = pack_bf16x2(fmaf(w3, __uint_as_float(b4[j] << 16), __uint_as_float(a[j] << 16)),
                          fmaf(w3, __uint_as_float(b4[j] & 0xffff0000u),
                               __uint_as_float(a[j] & 0xffff0000u)));
    vv = make_uint4(r4[0], r4[1], r4[2], r4[3]);
  }
  st16(vc + dst, vv);
}

hipError_t launch_kv_append_bf16(const void* k_new, const void* v_new, void* kc, void* vc,
                                 const int* lens, int B, int T, int Hk, int Tc,
                                 const float* cos_t, const float* sin_t, float eps,
                                 const void* ve, const void* gate, hipStream_t s) {
  const bool rope = cos_t != nullptr, gated = ve != nullptr;
  const long chunks = static_cast<long>(B) * T * Hk * D / 8;
  auto* append = rope ? (gated ? kv_append_kernel<true, true> : kv_append_kernel<true, false>)
                      : (gated ? kv_append_kernel<false, true> : kv_append_kernel<false, false>);
  return launch(append, dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0, s,
                static_cast<const u16*>(k_new), static_cast<const u16*>(v_new),
                static_cast<u16*>(kc), static_cast<u16*>(vc), lens, T, Tc, Hk, chunks, cos_t,
                sin_t, eps, static_cast<const u16*>(ve), static_cast<const u16*>(gate));
}

hipError_t launch_prefill_bf16(const void* q, const void* k_new, const void* v_new, void* kc,
                               void* vc, const int* lens, void* o, float* lse, int B, int T,
                               int H, int Hk, int Tc, int window, hipStream_t s,
                               const float* cos_t, const float* sin_t, float eps,
                               const void* ve, const void* gate) {
  const bool rope = cos_t != nullptr;
  hipError_t e = launch_kv_append_bf16(k_new, v_new, kc, vc, lens, B, T, Hk, Tc, cos_t, sin_t,
                                       eps, ve, gate, s);
  if (e != hipSuccess) return e;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float c_log2 = scale * 1.4426950408889634f;
  const int n_qt = (T + BQ - 1) / BQ;
  const dim3 grid(static_cast<unsigned>(n_qt) * B * H);
  const bool win = window >= 0 && window < Tc - 1;  // else every row sees all its keys
  auto* kern = rope ? (win ? fwd_bf16_kernel<true, true, true> : fwd_bf16_kernel<false, true, true>)
                    : (win ? fwd_bf16_kernel<true, true> : fwd_bf16_kernel<false, true>);
  return launch(kern, grid, dim3(64 * NW), 0, s, static_cast<const u16*>(q),
                static_cast<const u16*>(kc), static_cast<const u16*>(vc), static_cast<u16*>(o),
                lse, B, T, Tc, H, Hk, lens, c_log2, scale, win ? window : Tc, cos_t, sin_t, eps,
                static_cast<u16*>(nullptr));
}

}  // namespace na
