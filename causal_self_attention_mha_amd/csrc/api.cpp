// C-ABI layer of the attention library: host-side argument checks, then the
// kernel launches.  Every check runs before any HIP call, so a rejected call
// enqueues nothing and works without a GPU present.
#include "../../include/na_attn.h"
#include "internal.hpp"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

namespace {

thread_local char g_msg[256] = "";

na_status fail(na_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
na_status fail(na_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return st;
}

na_status ok() {
  g_msg[0] = '\0';
  return NA_OK;
}

na_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<std::uintptr_t>(p) & 15u) == 0; }

struct Ptr {
  const void* p;
  const char* name;
};

na_status check_ptrs(std::initializer_list<Ptr> ins, std::initializer_list<Ptr> outs) {
  for (auto l : {ins, outs})
    for (const Ptr& x : l) {
      if (x.p == nullptr) return fail(NA_ERR_INVALID_ARG, "%s is NULL", x.name);
      if (!aligned16(x.p)) return fail(NA_ERR_INVALID_ARG, "%s is not 16-byte aligned", x.name);
    }
  for (const Ptr& o : outs) {
    for (const Ptr& i : ins)
      if (o.p == i.p) return fail(NA_ERR_INVALID_ARG, "output %s aliases input %s", o.name, i.name);
    for (const Ptr& o2 : outs)
      if (&o2 != &o && o2.p == o.p)
        return fail(NA_ERR_INVALID_ARG, "outputs %s and %s alias", o.name, o2.name);
  }
  return NA_OK;
}

// Sizes of a (B, T, H, D) problem: all >= 1, D == 128, element count and the
// largest grid within what 64-bit indexing and HIP's grid limits allow.
na_status check_sizes(int B, int T, int H, int D) {
  if (B < 1 || T < 1 || H < 1 || D < 1)
    return fail(NA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d T=%d H=%d D=%d)", B, T, H, D);
  if (D != na::kHeadDim)
    return fail(NA_ERR_UNSUPPORTED, "head dim D=%d is not supported (only 128)", D);
  const long double n = (long double)B * T * H * D;
  if (n >= 9.2e18L) return fail(NA_ERR_INVALID_ARG, "B*T*H*D overflows 64-bit indexing");
  // kernels index rows of one batch with 32-bit offsets
  if ((long double)T * H * D > 2147483647.0L)
    return fail(NA_ERR_UNSUPPORTED, "T*H*D = %.0Lf per batch exceeds 2^31-1",
                (long double)T * H * D);
  // every grid is at most B*H*T workgroups in x
  if ((long double)B * H * T > 2147483647.0L)
    return fail(NA_ERR_INVALID_ARG, "B*H*T exceeds the launch grid limit");
  return NA_OK;
}

// Key/value heads: 1 <= H_kv <= H and H a multiple of H_kv.
na_status check_kv_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(NA_ERR_INVALID_ARG, "H=%d is not a multiple of H_kv=%d (1 <= H_kv <= H)", H,
                H_kv);
  return NA_OK;
}

}  // namespace

extern "C" {

const char* na_status_string(na_status s) {
  switch (s) {
    case NA_OK: return "NA_OK";
    case NA_ERR_INVALID_ARG: return "NA_ERR_INVALID_ARG: an argument failed a host-side check";
    case NA_ERR_UNSUPPORTED: return "NA_ERR_UNSUPPORTED: shape or option not supported";
    case NA_ERR_HIP: return "NA_ERR_HIP: a HIP launch failed";
    default: return "unknown na_status";
  }
}

const char* na_last_error(void) { return g_msg; }

na_status na_attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int T, int H, int H_kv, int D, int window, void* stream) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}}, {{o, "o"}, {lse, "lse"}});
  if (st) return st;
  return hip_status(
      na::launch_fwd_bf16(q, k, v, o, lse, B, T, H, H_kv, window, (hipStream_t)stream),
      "na_attn_fwd");
}

na_status na_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T, int H, int D, int window, void* stream) {
  return na_attn_fwd_gqa(q, k, v, o, lse, B, T, H, H, D, window, stream);
}

na_status na_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int T, int H, int D, void* stream) {
  return na_attn_fwd_window(q, k, v, o, lse, B, T, H, D, -1, stream);
}

na_status na_attn_prefill(const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, const int* cache_lens, void* o, float* lse, int B,
                          int T_q, int H, int H_kv, int D, int T_cap, int window,
                          void* stream) {
  na_status st = check_sizes(B, T_q, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  if (T_cap < T_q)
    return fail(NA_ERR_INVALID_ARG, "T_cap=%d is smaller than the chunk T_q=%d", T_cap, T_q);
  if ((st = check_sizes(B, T_cap, H, D))) return st;  // the caches' extent
  if (lse != nullptr)
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {cache_lens, "cache_lens"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"}, {lse, "lse"}});
  else
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {cache_lens, "cache_lens"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"}});
  if (st) return st;
  return hip_status(na::launch_prefill_bf16(q, k_new, v_new, k_cache, v_cache, cache_lens, o, lse,
                                            B, T_q, H, H_kv, T_cap, window,
                                            (hipStream_t)stream),
                    "na_attn_prefill");
}

na_status na_attn_prefill_rope(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const int* cache_lens,
                               const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                               const void* ve, const void* gate, void* o, float* lse, int B,
                               int T_q, int H, int H_kv, int D, int T_cap, int window,
                               void* stream) {
  na_status st = check_sizes(B, T_q, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  if (T_cap < T_q)
    return fail(NA_ERR_INVALID_ARG, "T_cap=%d is smaller than the chunk T_q=%d", T_cap, T_q);
  if ((st = check_sizes(B, T_cap, H, D))) return st;
  if (T_tab < T_cap)
    return fail(NA_ERR_INVALID_ARG, "T_tab=%d is smaller than T_cap=%d", T_tab, T_cap);
  if ((long double)T_tab * D > 2147483647.0L)
    return fail(NA_ERR_UNSUPPORTED, "the rotary tables (T_tab=%d) exceed 2^31-1 elements", T_tab);
  if (!(eps >= 0.f) || eps > 3.0e38f) return fail(NA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if ((ve == nullptr) != (gate == nullptr))
    return fail(NA_ERR_INVALID_ARG, "ve and gate are given together or not at all");
  if (ve != nullptr) {
    st = check_ptrs({{ve, "ve"}, {gate, "gate"}}, {{k_cache, "k_cache"}, {v_cache, "v_cache"},
                                                   {o, "o"}});
    if (st) return st;
  }
  if (lse != nullptr)
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {cache_lens, "cache_lens"},
                     {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"}, {lse, "lse"}});
  else
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {cache_lens, "cache_lens"},
                     {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"}});
  if (st) return st;
  return hip_status(na::launch_prefill_bf16(q, k_new, v_new, k_cache, v_cache, cache_lens, o, lse,
                                            B, T_q, H, H_kv, T_cap, window, (hipStream_t)stream,
                                            cos_tab, sin_tab, eps, ve, gate),
                    "na_attn_prefill_rope");
}

size_t na_attn_bwd_workspace_bytes(int B, int T, int H, int D) {
  if (B < 1 || T < 1 || H < 1 || D != na::kHeadDim || T > 1048576) return 0;
  return na::bwd_workspace_bytes(B, T, H);
}

na_status na_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* delta, void* workspace, size_t workspace_bytes, int B, int T,
                          int H, int H_kv, int D, int window, void* stream,
                          void* const* events) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  if (workspace != nullptr) {
    st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {dout, "dout"}, {lse, "lse"}},
                    {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {delta, "delta"},
                     {workspace, "workspace"}});
    if (st) return st;
    if (T > 1048576)
      return fail(NA_ERR_UNSUPPORTED, "the dS workspace path needs T <= 1048576 (T=%d)", T);
    const size_t need = na::bwd_workspace_bytes(B, T, H);
    if (workspace_bytes < need)
      return fail(NA_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", workspace_bytes,
                  need);
  } else {
    st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {dout, "dout"}, {lse, "lse"}},
                    {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {delta, "delta"}});
    if (st) return st;
  }
  return hip_status(na::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, workspace, B,
                                        T, H, H_kv, window, (hipStream_t)stream,
                                        reinterpret_cast<hipEvent_t const*>(events)),
                    "na_attn_bwd");
}

na_status na_attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, void* workspace, size_t workspace_bytes, int B,
                             int T, int H, int D, int window, void* stream,
                             void* const* events) {
  return na_attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, delta, workspace, workspace_bytes,
                         B, T, H, H, D, window, stream, events);
}

na_status na_attn_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* delta, void* workspace, size_t workspace_bytes, int B,
                            int T, int H, int D, void* stream, void* const* events) {
  return na_attn_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, delta, workspace,
                            workspace_bytes, B, T, H, D, -1, stream, events);
}

na_status na_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, void* workspace, size_t workspace_bytes, int B, int T,
                      int H, int D, void* stream) {
  return na_attn_bwd_timed(q, k, v, o, dout, lse, dq, dk, dv, delta, workspace, workspace_bytes,
                           B, T, H, D, stream, nullptr);
}

size_t na_attn_decode_workspace_bytes(int B, int H, int D, int T_cap) {
  if (B < 1 || H < 1 || T_cap < 1 || D != na::kHeadDim) return 0;
  return na::decode_workspace_bytes(B, H, T_cap);
}

na_status na_attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                             const int* seqlens, void* o, float* lse, int B, int H, int H_kv,
                             int D, int T_cap, int window, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events) {
  na_status st = check_sizes(B, T_cap, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  if (lse != nullptr) {
    st = check_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {seqlens, "seqlens"}},
                    {{o, "o"}, {lse, "lse"}, {workspace, "workspace"}});
  } else {
    st = check_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {seqlens, "seqlens"}},
                    {{o, "o"}, {workspace, "workspace"}});
  }
  if (st) return st;
  if (B > 65535) return fail(NA_ERR_INVALID_ARG, "decode supports B <= 65535 (B=%d)", B);
  if (H > 32) return fail(NA_ERR_UNSUPPORTED, "decode supports H <= 32 (H=%d)", H);
  const size_t need = na::decode_workspace_bytes(B, H, T_cap);
  if (workspace_bytes < need)
    return fail(NA_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  return hip_status(na::launch_decode_bf16(q, k_cache, v_cache, seqlens, o, lse, B, H, H_kv,
                                           T_cap, window, workspace, (hipStream_t)stream,
                                           reinterpret_cast<hipEvent_t const*>(events)),
                    "na_attn_decode");
}

na_status na_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const void* q_raw,
                           const void* k_raw, const float* cos_tab, const float* sin_tab,
                           int T_tab, float eps, const void* ve, const void* gate, void* dq,
                           void* dk, void* dv, void* dve, void* dgate, float* delta,
                           void* workspace, size_t workspace_bytes, int B, int T, int H,
                           int H_kv, int D, int window, void* stream) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {dout, "dout"}, {lse, "lse"},
                   {q_raw, "q_raw"}, {k_raw, "k_raw"}, {cos_tab, "cos_tab"},
                   {sin_tab, "sin_tab"}},
                  {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {delta, "delta"},
                   {workspace, "workspace"}});
  if (st) return st;
  const int n_gate = (ve != nullptr) + (gate != nullptr) + (dve != nullptr) + (dgate != nullptr);
  if (n_gate != 0 && n_gate != 4)
    return fail(NA_ERR_INVALID_ARG, "ve, gate, dve, dgate: give all four or none");
  if (n_gate == 4 && (dve == dv || dve == dk || dve == dq || dgate == dv || dgate == dve))
    return fail(NA_ERR_INVALID_ARG, "dve and dgate must not alias another output");
  if (T_tab < T) return fail(NA_ERR_INVALID_ARG, "T_tab=%d is smaller than T=%d", T_tab, T);
  if ((long double)T_tab * D > 2147483647.0L)
    return fail(NA_ERR_UNSUPPORTED, "the rotary tables (T_tab=%d) exceed 2^31-1 elements", T_tab);
  if (!(eps >= 0.f) || eps > 3.0e38f) return fail(NA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (T > 1048576)
    return fail(NA_ERR_UNSUPPORTED, "the dS workspace path needs T <= 1048576 (T=%d)", T);
  const size_t need = na::bwd_workspace_bytes(B, T, H);
  if (workspace_bytes < need)
    return fail(NA_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  return hip_status(na::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, workspace, B, T,
                                        H, H_kv, window, (hipStream_t)stream, nullptr, q_raw,
                                        k_raw, cos_tab, sin_tab, eps, ve, gate, dve, dgate),
                    "na_attn_bwd_rope");
}

na_status na_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int* seqlens,
                                const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                                const void* ve, const void* gate, void* o, float* lse, int B,
                                int H, int H_kv, int D, int T_cap, int window, void* workspace,
                                size_t workspace_bytes, void* stream) {
  na_status st = check_sizes(B, T_cap, H, D);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  if (lse != nullptr)
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {seqlens, "seqlens"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"}, {lse, "lse"},
                     {workspace, "workspace"}});
  else
    st = check_ptrs({{q, "q"}, {k_new, "k_new"}, {v_new, "v_new"}, {seqlens, "seqlens"}},
                    {{k_cache, "k_cache"}, {v_cache, "v_cache"}, {o, "o"},
                     {workspace, "workspace"}});
  if (st) return st;
  if ((cos_tab == nullptr) != (sin_tab == nullptr))
    return fail(NA_ERR_INVALID_ARG, "cos_tab and sin_tab are given together or not at all");
  if (cos_tab != nullptr) {
    if ((st = check_ptrs({{cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}}, {{o, "o"}}))) return st;
    if (T_tab < T_cap)
      return fail(NA_ERR_INVALID_ARG, "T_tab=%d is smaller than T_cap=%d", T_tab, T_cap);
    if ((long double)T_tab * D > 2147483647.0L)
      return fail(NA_ERR_UNSUPPORTED, "the rotary tables (T_tab=%d) exceed 2^31-1 elements",
                  T_tab);
    if (!(eps >= 0.f) || eps > 3.0e38f)
      return fail(NA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  }
  if ((ve == nullptr) != (gate == nullptr))
    return fail(NA_ERR_INVALID_ARG, "ve and gate are given together or not at all");
  if (ve != nullptr && (st = check_ptrs({{ve, "ve"}, {gate, "gate"}}, {{o, "o"}}))) return st;
  if (B > 65535) return fail(NA_ERR_INVALID_ARG, "decode supports B <= 65535 (B=%d)", B);
  if (H > 32) return fail(NA_ERR_UNSUPPORTED, "decode supports H <= 32 (H=%d)", H);
  const size_t need = na::decode_workspace_bytes(B, H, T_cap);
  if (workspace_bytes < need)
    return fail(NA_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  return hip_status(na::launch_decode_bf16(q, k_cache, v_cache, seqlens, o, lse, B, H, H_kv,
                                           T_cap, window, workspace, (hipStream_t)stream, nullptr,
                                           k_new, v_new, cos_tab, sin_tab, eps, ve, gate),
                    "na_attn_decode_append");
}

na_status na_attn_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                const int* seqlens, void* o, float* lse, int B, int H, int D,
                                int T_cap, int window, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* events) {
  return na_attn_decode_gqa(q, k_cache, v_cache, seqlens, o, lse, B, H, H, D, T_cap, window,
                            workspace, workspace_bytes, stream, events);
}

na_status na_attn_decode_timed(const void* q, const void* k_cache, const void* v_cache,
                               const int* seqlens, void* o, float* lse, int B, int H, int D,
                               int T_cap, void* workspace, size_t workspace_bytes, void* stream,
                               void* const* events) {
  return na_attn_decode_window(q, k_cache, v_cache, seqlens, o, lse, B, H, D, T_cap, -1,
                               workspace, workspace_bytes, stream, events);
}

na_status na_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int* seqlens, void* o, float* lse, int B, int H, int D,
                         int T_cap, void* workspace, size_t workspace_bytes, void* stream) {
  return na_attn_decode_timed(q, k_cache, v_cache, seqlens, o, lse, B, H, D, T_cap, workspace,
                              workspace_bytes, stream, nullptr);
}

na_status na_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seqlens, void* o, float* lse, int B, int H, int D,
                                 int T_cap, void* stream) {
  na_status st = check_sizes(B, T_cap, H, D);
  if (st) return st;
  if (lse != nullptr) {
    st = check_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {seqlens, "seqlens"}},
                    {{o, "o"}, {lse, "lse"}});
  } else {
    st = check_ptrs({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {seqlens, "seqlens"}},
                    {{o, "o"}});
  }
  if (st) return st;
  if (B > 65535) return fail(NA_ERR_INVALID_ARG, "decode supports B <= 65535 (B=%d)", B);
  if (H > 32) return fail(NA_ERR_UNSUPPORTED, "decode supports H <= 32 (H=%d)", H);
  const size_t need = na::decode_workspace_bytes(B, H, T_cap);
  if (need > na::kDecodeScratchBytes)
    return fail(NA_ERR_INVALID_ARG,
                "these sizes need %zu bytes of decode scratch; the library's own scratch holds "
                "%zu (pass a workspace to na_attn_decode instead)",
                need, na::kDecodeScratchBytes);
  void* ws = nullptr;
  if (hipError_t e = na::decode_scratch(&ws); e != hipSuccess)
    return hip_status(e, "na_attn_decode_noalloc (scratch lookup)");
  return hip_status(na::launch_decode_bf16(q, k_cache, v_cache, seqlens, o, lse, B, H, H, T_cap,
                                           -1, ws, (hipStream_t)stream, nullptr),
                    "na_attn_decode_noalloc");
}

na_status na_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int T, int H, int D, void* stream) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}}, {{o, "o"}, {lse, "lse"}});
  if (st) return st;
  return hip_status(na::launch_fwd_f32(q, k, v, o, lse, B, T, H, (hipStream_t)stream),
                    "na_attn_fwd_f32");
}

na_status na_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int T, int H, int D, void* stream) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {dout, "dout"}, {lse, "lse"}},
                  {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {delta, "delta"}});
  if (st) return st;
  return hip_status(na::launch_bwd_f32(q, k, v, o, dout, lse, dq, dk, dv, delta, B, T, H,
                                       (hipStream_t)stream),
                    "na_attn_bwd_f32");
}

}  // extern "C"

namespace {

na_status check_prologue(int B, int T, int H, int H_kv, int D, int T_tab, float eps) {
  na_status st = check_sizes(B, T, H, D);
  if (st) return st;
  if ((st = check_sizes(B, T, H_kv, D))) return st;
  if (T_tab < T) return fail(NA_ERR_INVALID_ARG, "T_tab=%d is smaller than T=%d", T_tab, T);
  if ((long double)T_tab * D > 2147483647.0L)
    return fail(NA_ERR_UNSUPPORTED, "the rotary tables (T_tab=%d) exceed 2^31-1 elements", T_tab);
  if (!(eps >= 0.f) || eps > 3.0e38f)
    return fail(NA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return NA_OK;
}

}  // namespace

extern "C" {

na_status na_qk_norm_rope_fwd(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, const int* pos_offset,
                              int B, int T, int H, int H_kv, int D, int T_tab, float eps,
                              void* stream) {
  na_status st = check_prologue(B, T, H, H_kv, D, T_tab, eps);
  if (st) return st;
  if (pos_offset != nullptr)
    st = check_ptrs({{q, "q"}, {k, "k"}, {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"},
                     {pos_offset, "pos_offset"}},
                    {{q_out, "q_out"}, {k_out, "k_out"}});
  else
    st = check_ptrs({{q, "q"}, {k, "k"}, {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}},
                    {{q_out, "q_out"}, {k_out, "k_out"}});
  if (st) return st;
  return hip_status(na::launch_qk_norm_rope_bf16(q, k, nullptr, nullptr, q_out, k_out, cos_tab,
                                                 sin_tab, pos_offset, B, T, H, H_kv, T_tab, eps,
                                                 false, (hipStream_t)stream),
                    "na_qk_norm_rope_fwd");
}

na_status na_attn_fwd_rope(const void* q_raw, const void* k_raw, const void* v,
                           const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                           void* q_rot, void* k_rot, void* o, float* lse, int B, int T, int H,
                           int H_kv, int D, int window, void* stream) {
  na_status st = check_prologue(B, T, H, H_kv, D, T_tab, eps);
  if (st) return st;
  if ((st = check_kv_heads(H, H_kv))) return st;
  st = check_ptrs({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v, "v"}, {cos_tab, "cos_tab"},
                   {sin_tab, "sin_tab"}},
                  {{q_rot, "q_rot"}, {k_rot, "k_rot"}, {o, "o"}, {lse, "lse"}});
  if (st) return st;
  hipError_t e = na::launch_qk_norm_rope_bf16(nullptr, k_raw, nullptr, nullptr, nullptr, k_rot,
                                              cos_tab, sin_tab, nullptr, B, T, H, H_kv, T_tab,
                                              eps, false, (hipStream_t)stream);
  if (e == hipSuccess)
    e = na::launch_fwd_bf16(q_raw, k_rot, v, o, lse, B, T, H, H_kv, window, (hipStream_t)stream,
                            cos_tab, sin_tab, eps, q_rot);
  return hip_status(e, "na_attn_fwd_rope");
}

na_status na_qk_norm_rope_bwd(const void* q, const void* k, const void* dq_rot,
                              const void* dk_rot, void* dq, void* dk, const float* cos_tab,
                              const float* sin_tab, const int* pos_offset, int B, int T, int H,
                              int H_kv, int D, int T_tab, float eps, void* stream) {
  na_status st = check_prologue(B, T, H, H_kv, D, T_tab, eps);
  if (st) return st;
  if (pos_offset != nullptr)
    st = check_ptrs({{q, "q"}, {k, "k"}, {dq_rot, "dq_rot"}, {dk_rot, "dk_rot"},
                     {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}, {pos_offset, "pos_offset"}},
                    {{dq, "dq"}, {dk, "dk"}});
  else
    st = check_ptrs({{q, "q"}, {k, "k"}, {dq_rot, "dq_rot"}, {dk_rot, "dk_rot"},
                     {cos_tab, "cos_tab"}, {sin_tab, "sin_tab"}},
                    {{dq, "dq"}, {dk, "dk"}});
  if (st) return st;
  return hip_status(na::launch_qk_norm_rope_bf16(q, k, dq_rot, dk_rot, dq, dk, cos_tab, sin_tab,
                                                 pos_offset, B, T, H, H_kv, T_tab, eps, true,
                                                 (hipStream_t)stream),
                    "na_qk_norm_rope_bwd");
}

na_status na_value_gate_fwd(const void* v, const void* ve, const void* gate, void* v_out, int B,
                            int T, int H_kv, int D, void* stream) {
  na_status st = check_sizes(B, T, H_kv, D);
  if (st) return st;
  st = check_ptrs({{v, "v"}, {ve, "ve"}, {gate, "gate"}}, {{v_out, "v_out"}});
  if (st) return st;
  return hip_status(na::launch_value_gate_bf16(v, ve, gate, v_out, nullptr, B, T, H_kv, false,
                                               (hipStream_t)stream),
                    "na_value_gate_fwd");
}

na_status na_value_gate_bwd(const void* ve, const void* gate, const void* dv_out, void* dve,
                            void* dgate, int B, int T, int H_kv, int D, void* stream) {
  na_status st = check_sizes(B, T, H_kv, D);
  if (st) return st;
  st = check_ptrs({{ve, "ve"}, {gate, "gate"}, {dv_out, "dv_out"}},
                  {{dve, "dve"}, {dgate, "dgate"}});
  if (st) return st;
  return hip_status(na::launch_value_gate_bf16(dv_out, ve, gate, dve, dgate, B, T, H_kv, true,
                                               (hipStream_t)stream),
                    "na_value_gate_bwd");
}

}  // extern "C"
