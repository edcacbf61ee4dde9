// C ABI of the attention library: argument validation, workspace sizing,
// cu_seqlens checking on request, and kernel dispatch. Every check that can be
// made on the host runs before any HIP call, so invalid calls fail without a
// GPU and without launching anything.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "attn_error.hpp"
#include "attn_launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int ok() { return ATTN_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int dtype, int Hq, int Hkv, int Dqk, int Dv, float scale) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_E_UNSUPPORTED, "dtype must be ATTN_BF16 or ATTN_F16");
  if (Hq <= 0 || Hkv <= 0) return fail(ATTN_E_INVALID, "Hq and Hkv must be positive");
  if (Hq % Hkv != 0) return fail(ATTN_E_INVALID, "Hq must be a multiple of Hkv (GQA)");
  if (!vca::head_dims_supported(Dqk, Dv))
    return fail(ATTN_E_UNSUPPORTED, "head dims (" + std::to_string(Dqk) + "," +
                                        std::to_string(Dv) + ") not compiled in");
  if (!std::isfinite(scale) || scale == 0.f)
    return fail(ATTN_E_INVALID, "scale must be finite and non-zero");
  return ATTN_OK;
}

int check_tensor(const char* name, const void* p, bool nonempty, const int64_t* strides, int n) {
  if (nonempty && p == nullptr) return fail(ATTN_E_INVALID, std::string(name) + " is NULL");
  if (p && !aligned16(p)) return fail(ATTN_E_INVALID, std::string(name) + " is not 16-byte aligned");
  for (int i = 0; i < n; ++i) {
    if (strides[i] < 0 || strides[i] % 8 != 0)
      return fail(ATTN_E_INVALID, std::string(name) + " strides must be non-negative multiples of 8");
  }
  return ATTN_OK;
}

// workspace protocol: (workspace == NULL && workspace_bytes != NULL) is a size
// query; otherwise a call that needs `need` bytes must be given them.
int workspace_step(size_t need, void* ws, size_t* ws_bytes, bool* query) {
  *query = false;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    *query = true;
    return ATTN_OK;
  }
  if (need == 0) return ATTN_OK;
  if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < need)
    return fail(ATTN_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  if (!aligned16(ws)) return fail(ATTN_E_INVALID, "workspace is not 16-byte aligned");
  return ATTN_OK;
}

bool validate_env() {
  const char* e = std::getenv("ATTN_VALIDATE");
  return e && e[0] == '1';
}

// Host copy of cu_seqlens and a full contract check (ATTN_VALIDATE=1 only).
int validate_cu(const int32_t* cu_q, const int32_t* cu_k, int S, int Tq, int Tk, int max_q,
                int max_k, hipStream_t st) {
  std::vector<int32_t> hq(S + 1), hk(S + 1);
  hipError_t e = hipMemcpyAsync(hq.data(), cu_q, sizeof(int32_t) * (S + 1), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(hk.data(), cu_k, sizeof(int32_t) * (S + 1), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("cu_seqlens copy: ") + hipGetErrorString(e));
  if (hq[0] != 0 || hk[0] != 0) return fail(ATTN_E_INVALID, "cu_seqlens must start at 0");
  if (hq[S] != Tq || hk[S] != Tk) return fail(ATTN_E_INVALID, "cu_seqlens must end at Tq / Tk");
  for (int s = 0; s < S; ++s) {
    const int lq = hq[s + 1] - hq[s], lk = hk[s + 1] - hk[s];
    if (lq < 0 || lk < 0) return fail(ATTN_E_INVALID, "cu_seqlens must be non-decreasing");
    if (lq > max_q || lk > max_k) return fail(ATTN_E_INVALID, "segment longer than max_q / max_k");
  }
  return ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The kernels of the call's element type (validated by check_heads).
auto fwd_launcher(int dtype) { return dtype == ATTN_F16 ? vca::hf::launch_fwd : vca::bf::launch_fwd; }
auto bwd_launcher(int dtype) { return dtype == ATTN_F16 ? vca::hf::launch_bwd : vca::bf::launch_bwd; }

vca::View view(const void* p, int64_t sb, int64_t sh, int64_t sn) {
  return vca::View{static_cast<const uint16_t*>(p), sb, sh, sn};
}
vca::ViewW vieww(void* p, int64_t sb, int64_t sh, int64_t sn) {
  return vca::ViewW{static_cast<uint16_t*>(p), sb, sh, sn};
}

// Window / softcap options: 0 = off. The window needs the causal mask; both
// must be non-negative and finite.
int check_ext(const attn_ext* ext, int causal) {
  if (!ext) return ATTN_OK;
  if (ext->window < 0) return fail(ATTN_E_INVALID, "window must be >= 0");
  if (ext->window > 0 && !causal) return fail(ATTN_E_INVALID, "a window needs causal = 1");
  if (!(ext->softcap >= 0.f) || std::isinf(ext->softcap))
    return fail(ATTN_E_INVALID, "softcap must be finite and >= 0");
  return ATTN_OK;
}
// Kernel fields of the options. The forward folds a negative scale into Q and
// works on scale * q.k as |scale| * s, so its tanh argument factor is
// |scale| / cap; the backward's scores are raw q.k, so its factor is
// scale / cap. cap_out = cap * log2(e) puts the capped score in base-2 units.
template <class Args>
void set_ext(Args& a, const attn_ext* ext, float scale, bool fwd) {
  a.window = ext ? ext->window : 0;
  const float cap = ext ? ext->softcap : 0.f;
  a.cap_in = cap > 0.f ? (fwd ? std::fabs(scale) : scale) / cap : 0.f;
  a.cap_out = cap > 0.f ? cap * vca::kLog2e : 0.f;
}

// Argument checks of the varlen forward (everything visible on the host).
int fwd_varlen_checks(int dtype, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const int32_t* cu_q, const int32_t* cu_k,
                      int num_segments, int max_q, int max_k, int Tq, int Tk, int Hq, int Hkv,
                      int Dqk, int Dv, const int64_t* strides, float scale) {
  int st = check_heads(dtype, Hq, Hkv, Dqk, Dv, scale);
  if (st) return st;
  if (num_segments < 0 || Tq < 0 || Tk < 0 || max_q < 0 || max_k < 0)
    return fail(ATTN_E_INVALID, "sizes must be >= 0");
  if (!strides) return fail(ATTN_E_INVALID, "strides is NULL");
  if (num_segments > 0 && (!cu_q || !cu_k)) return fail(ATTN_E_INVALID, "cu_seqlens is NULL");
  if (num_segments == 0 && (Tq > 0 || Tk > 0))
    return fail(ATTN_E_INVALID, "tokens given but no segments");
  if (Tq > 0 && max_q < 1) return fail(ATTN_E_INVALID, "max_q must be >= 1 when Tq > 0");
  if (Tk > 0 && max_k < 1) return fail(ATTN_E_INVALID, "max_k must be >= 1 when Tk > 0");
  if ((st = check_tensor("q", q, Tq > 0, strides + 0, 2))) return st;
  if ((st = check_tensor("k", k, Tk > 0, strides + 2, 2))) return st;
  if ((st = check_tensor("v", v, Tk > 0, strides + 4, 2))) return st;
  if ((st = check_tensor("out", out, Tq > 0, strides + 6, 2))) return st;
  if (Tq > 0 && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
  return ATTN_OK;
}

// The varlen forward on checked arguments with a workspace of at least
// fwd_workspace_bytes (the scheduler writes every byte it later reads).
int fwd_varlen_run(int dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                   const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                   int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                   const int64_t* strides, float scale, int causal, const attn_ext* ext,
                   void* ws, hipStream_t stream, const char* what) {
  int st;
  if (validate_env() && (st = validate_cu(cu_q, cu_k, num_segments, Tq, Tk, max_q, max_k, stream)))
    return st;
  vca::FwdArgs a{};
  a.q = view(q, 0, strides[1], strides[0]);
  a.k = view(k, 0, strides[3], strides[2]);
  a.v = view(v, 0, strides[5], strides[4]);
  a.o = vieww(out, 0, strides[7], strides[6]);
  a.lse = lse;
  a.lse_sb = 0;
  a.lse_sh = Tq;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.Nq = a.Nk = 0;
  a.Tq = Tq;
  a.Tk = Tk;
  a.G = Hq / Hkv;
  a.scale_log2 = scale * vca::kLog2e;
  set_ext(a, ext, scale, true);
  return hip_status(
      fwd_launcher(dtype)(a, Dqk, Dv, causal != 0, num_segments, Hq, Tq, ws, stream), what);
}

// Static scratch of attn_fwd_varlen_noalloc: the forward's work list lives in
// this device array (one copy per GPU, held until the process ends) instead
// of a caller workspace. Host code never passes the array's name to a kernel
// (on the host it only stands in for the symbol): each device's address is
// taken with hipGetSymbolAddress on its first call there, with that device
// current, and kept.
constexpr size_t kScratchBytes = size_t(4) << 20;
static_assert(kScratchBytes == 256 + ATTN_NOALLOC_MAX_ITEMS * 8, "scratch size vs header");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_E_INVALID, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ATTN_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

void vca::set_last_error(const std::string& msg) { g_last_error = msg; }

bool vca::head_dims_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128) ||
         (dqk == 256 && dv == 256) || (dqk == 512 && dv == 512);
}

namespace {
// A MiB count from the environment (non-negative integer), else the default.
size_t env_mib(const char* name, long long dflt) {
  const char* e = std::getenv(name);
  long long mib = dflt;
  if (e && *e) {
    char* end = nullptr;
    const long long v = std::strtoll(e, &end, 10);
    if (end && *end == '\0' && v >= 0) mib = v;
  }
  return (size_t)mib << 20;
}
}  // namespace

size_t vca::ds_budget_bytes() { return env_mib("ATTN_BWD_DS_MIB", 8192); }
size_t vca::tiles_budget_bytes() { return env_mib("ATTN_BWD_TILES_MIB", 8192); }


extern "C" {

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_version(void) { return 10000; }

int attn_is_supported(int dtype, int dqk, int dv) {
  return (dtype == ATTN_BF16 || dtype == ATTN_F16) && vca::head_dims_supported(dqk, dv) ? 1 : 0;
}

int attn_fwd_dense(int dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv, const int64_t* strides,
                   float scale, int causal, void* workspace, size_t* workspace_bytes,
                   hipStream_t stream) {
  return attn_fwd_dense_ex(dtype, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, Dqk, Dv, strides, scale,
                           causal, nullptr, workspace, workspace_bytes, stream);
}

int attn_fwd_dense_ex(int dtype, const void* q, const void* k, const void* v, void* out,
                      float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv,
                      const int64_t* strides, float scale, int causal, const attn_ext* ext,
                      void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_heads(dtype, Hq, Hkv, Dqk, Dv, scale);
  if (st) return st;
  if ((st = check_ext(ext, causal))) return st;
  if (B < 0 || Nq < 0 || Nk < 0) return fail(ATTN_E_INVALID, "B, Nq, Nk must be >= 0");
  if (!strides) return fail(ATTN_E_INVALID, "strides is NULL");
  const bool has_q = (int64_t)B * Nq > 0, has_k = (int64_t)B * Nk > 0;
  if ((st = check_tensor("q", q, has_q, strides + 0, 3))) return st;
  if ((st = check_tensor("k", k, has_k, strides + 3, 3))) return st;
  if ((st = check_tensor("v", v, has_k, strides + 6, 3))) return st;
  if ((st = check_tensor("out", out, has_q, strides + 9, 3))) return st;
  if (has_q && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
  bool query = false;
  const size_t need_ws = vca::fwd_workspace_bytes((int64_t)B * Nq, B);
  if ((st = workspace_step(need_ws, workspace, workspace_bytes, &query))) return st;
  if (query || !has_q) return ok();

  vca::FwdArgs a{};
  a.q = view(q, strides[0], strides[1], strides[2]);
  a.k = view(k, strides[3], strides[4], strides[5]);
  a.v = view(v, strides[6], strides[7], strides[8]);
  a.o = vieww(out, strides[9], strides[10], strides[11]);
  a.lse = lse;
  a.lse_sb = (int64_t)Hq * Nq;
  a.lse_sh = Nq;
  a.cu_q = a.cu_k = nullptr;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Tq = Nq;
  a.Tk = Nk;
  a.G = Hq / Hkv;
  a.scale_log2 = scale * vca::kLog2e;
  set_ext(a, ext, scale, true);
  return hip_status(
      fwd_launcher(dtype)(a, Dqk, Dv, causal != 0, B, Hq, (int64_t)B * Nq, workspace, stream),
      "attn_fwd_dense launch");
}

int attn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                    int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                    const int64_t* strides, float scale, int causal, void* workspace,
                    size_t* workspace_bytes, hipStream_t stream) {
  return attn_fwd_varlen_ex(dtype, q, k, v, out, lse, cu_q, cu_k, num_segments, max_q, max_k, Tq,
                            Tk, Hq, Hkv, Dqk, Dv, strides, scale, causal, nullptr, workspace,
                            workspace_bytes, stream);
}

int attn_fwd_varlen_ex(int dtype, const void* q, const void* k, const void* v, void* out,
                       float* lse, const int32_t* cu_q, const int32_t* cu_k, int num_segments,
                       int max_q, int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                       const int64_t* strides, float scale, int causal, const attn_ext* ext,
                       void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = fwd_varlen_checks(dtype, q, k, v, out, lse, cu_q, cu_k, num_segments, max_q, max_k, Tq,
                             Tk, Hq, Hkv, Dqk, Dv, strides, scale);
  if (st) return st;
  if ((st = check_ext(ext, causal))) return st;
  bool query = false;
  const size_t need_ws = vca::fwd_workspace_bytes(Tq, num_segments);
  if ((st = workspace_step(need_ws, workspace, workspace_bytes, &query))) return st;
  if (query || Tq == 0) return ok();
  return fwd_varlen_run(dtype, q, k, v, out, lse, cu_q, cu_k, num_segments, max_q, max_k, Tq, Tk,
                        Hq, Hkv, Dqk, Dv, strides, scale, causal, ext, workspace, stream,
                        "attn_fwd_varlen launch");
}

int attn_fwd_varlen_noalloc(int dtype, const void* q, const void* k, const void* v, void* out,
                            float* lse, const int32_t* cu_q, const int32_t* cu_k,
                            int num_segments, int max_q, int max_k, int Tq, int Tk, int Hq,
                            int Hkv, int Dqk, int Dv, const int64_t* strides, float scale,
                            int causal, hipStream_t stream) {
  g_last_error.clear();
  int st = fwd_varlen_checks(dtype, q, k, v, out, lse, cu_q, cu_k, num_segments, max_q, max_k, Tq,
                             Tk, Hq, Hkv, Dqk, Dv, strides, scale);
  if (st) return st;
  const size_t need_ws = vca::fwd_workspace_bytes(Tq, num_segments);
  if (need_ws > kScratchBytes)
    return fail(ATTN_E_WORKSPACE, "attn_fwd_varlen_noalloc: the work list needs " +
                                      std::to_string(need_ws) + " bytes, the static scratch holds " +
                                      std::to_string(kScratchBytes) +
                                      " (at most ATTN_NOALLOC_MAX_ITEMS query tiles + segments)");
  if (Tq == 0) return ok();
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return fwd_varlen_run(dtype, q, k, v, out, lse, cu_q, cu_k, num_segments, max_q, max_k, Tq, Tk,
                        Hq, Hkv, Dqk, Dv, strides, scale, causal, nullptr, ws, stream,
                        "attn_fwd_varlen_noalloc launch");
}

int attn_bwd_dense(int dtype, const void* dout, const void* q, const void* k, const void* v,
                   const void* out, const float* lse, void* dq, void* dk, void* dv, int B, int Hq,
                   int Hkv, int Nq, int Nk, int Dqk, int Dv, const int64_t* strides, float scale,
                   int causal, int flags, void* workspace, size_t* workspace_bytes,
                   hipStream_t stream) {
  return attn_bwd_dense_ex(dtype, dout, q, k, v, out, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, Dqk, Dv,
                           strides, scale, causal, nullptr, flags, workspace, workspace_bytes,
                           stream);
}

int attn_bwd_dense_ex(int dtype, const void* dout, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, void* dq, void* dk, void* dv, int B,
                      int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv, const int64_t* strides,
                      float scale, int causal, const attn_ext* ext, int flags, void* workspace,
                      size_t* workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_heads(dtype, Hq, Hkv, Dqk, Dv, scale);
  if (st) return st;
  if ((st = check_ext(ext, causal))) return st;
  if (B < 0 || Nq < 0 || Nk < 0) return fail(ATTN_E_INVALID, "B, Nq, Nk must be >= 0");
  if (flags & ~ATTN_DQ_ACCUMULATE) return fail(ATTN_E_INVALID, "unknown flags");
  if (!strides) return fail(ATTN_E_INVALID, "strides is NULL");
  const bool has_q = (int64_t)B * Nq > 0, has_k = (int64_t)B * Nk > 0;
  const char* names[8] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
  const void* ptrs[8] = {q, k, v, out, dout, dq, dk, dv};
  const bool need[8] = {has_q, has_k, has_k, has_q, has_q, has_q, has_k, has_k};
  for (int i = 0; i < 8; ++i)
    if ((st = check_tensor(names[i], ptrs[i], need[i], strides + 3 * i, 3))) return st;
  if (has_q && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
  const vca::TileGeom tg = vca::tile_geom_dense(B, Nq, Nk);
  const size_t need_ws =
      vca::bwd_workspace(Dqk, Dv, Hq, Hkv, (int64_t)B * Nq, (int64_t)B * Nk, B, tg).total;
  bool query = false;
  if ((st = workspace_step(need_ws, workspace, workspace_bytes, &query))) return st;
  if (query || (!has_q && !has_k)) return ok();

  vca::BwdArgs a{};
  a.q = view(q, strides[0], strides[1], strides[2]);
  a.k = view(k, strides[3], strides[4], strides[5]);
  a.v = view(v, strides[6], strides[7], strides[8]);
  a.o = view(out, strides[9], strides[10], strides[11]);
  a.dout = view(dout, strides[12], strides[13], strides[14]);
  a.dq = vieww(dq, strides[15], strides[16], strides[17]);
  a.dk = vieww(dk, strides[18], strides[19], strides[20]);
  a.dv = vieww(dv, strides[21], strides[22], strides[23]);
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.lse_sb = (int64_t)Hq * Nq;
  a.lse_sh = Nq;
  a.cu_q = a.cu_k = nullptr;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Tq = Nq;
  a.Tk = Nk;
  a.G = Hq / Hkv;
  a.scale = scale;
  a.scale_log2 = scale * vca::kLog2e;
  a.inv_scale = 1.f / scale;
  a.dq_accumulate = (flags & ATTN_DQ_ACCUMULATE) ? 1 : 0;
  set_ext(a, ext, scale, false);
  return hip_status(bwd_launcher(dtype)(a, Dqk, Dv, causal != 0, B, Hq, Hkv, Nq, (int64_t)B * Nq,
                                        (int64_t)B * Nk, tg, workspace, stream),
                    "attn_bwd_dense launch");
}

int attn_bwd_varlen(int dtype, const void* dout, const void* q, const void* k, const void* v,
                    const void* out, const float* lse, void* dq, void* dk, void* dv,
                    const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                    int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                    const int64_t* strides, float scale, int causal, int flags, void* workspace,
                    size_t* workspace_bytes, hipStream_t stream) {
  return attn_bwd_varlen_ex(dtype, dout, q, k, v, out, lse, dq, dk, dv, cu_q, cu_k, num_segments,
                            max_q, max_k, Tq, Tk, Hq, Hkv, Dqk, Dv, strides, scale, causal,
                            nullptr, flags, workspace, workspace_bytes, stream);
}

int attn_bwd_varlen_ex(int dtype, const void* dout, const void* q, const void* k, const void* v,
                       const void* out, const float* lse, void* dq, void* dk, void* dv,
                       const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                       int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                       const int64_t* strides, float scale, int causal, const attn_ext* ext,
                       int flags, void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_heads(dtype, Hq, Hkv, Dqk, Dv, scale);
  if (st) return st;
  if ((st = check_ext(ext, causal))) return st;
  if (num_segments < 0 || Tq < 0 || Tk < 0 || max_q < 0 || max_k < 0)
    return fail(ATTN_E_INVALID, "sizes must be >= 0");
  if (flags & ~ATTN_DQ_ACCUMULATE) return fail(ATTN_E_INVALID, "unknown flags");
  if (!strides) return fail(ATTN_E_INVALID, "strides is NULL");
  if (num_segments > 0 && (!cu_q || !cu_k)) return fail(ATTN_E_INVALID, "cu_seqlens is NULL");
  if (num_segments == 0 && (Tq > 0 || Tk > 0))
    return fail(ATTN_E_INVALID, "tokens given but no segments");
  if (Tq > 0 && max_q < 1) return fail(ATTN_E_INVALID, "max_q must be >= 1 when Tq > 0");
  if (Tk > 0 && max_k < 1) return fail(ATTN_E_INVALID, "max_k must be >= 1 when Tk > 0");
  const char* names[8] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
  const void* ptrs[8] = {q, k, v, out, dout, dq, dk, dv};
  const bool need[8] = {Tq > 0, Tk > 0, Tk > 0, Tq > 0, Tq > 0, Tq > 0, Tk > 0, Tk > 0};
  for (int i = 0; i < 8; ++i)
    if ((st = check_tensor(names[i], ptrs[i], need[i], strides + 2 * i, 2))) return st;
  if (Tq > 0 && !lse) return fail(ATTN_E_INVALID, "lse is NULL");
  const vca::TileGeom tg = vca::tile_geom_varlen(Tq, num_segments, max_k);
  const size_t need_ws = vca::bwd_workspace(Dqk, Dv, Hq, Hkv, Tq, Tk, num_segments, tg).total;
  bool query = false;
  if ((st = workspace_step(need_ws, workspace, workspace_bytes, &query))) return st;
  if (query || (Tq == 0 && Tk == 0)) return ok();
  if (validate_env() && (st = validate_cu(cu_q, cu_k, num_segments, Tq, Tk, max_q, max_k, stream)))
    return st;

  vca::BwdArgs a{};
  a.q = view(q, 0, strides[1], strides[0]);
  a.k = view(k, 0, strides[3], strides[2]);
  a.v = view(v, 0, strides[5], strides[4]);
  a.o = view(out, 0, strides[7], strides[6]);
  a.dout = view(dout, 0, strides[9], strides[8]);
  a.dq = vieww(dq, 0, strides[11], strides[10]);
  a.dk = vieww(dk, 0, strides[13], strides[12]);
  a.dv = vieww(dv, 0, strides[15], strides[14]);
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.lse_sb = 0;
  a.lse_sh = Tq;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.Nq = a.Nk = 0;
  a.Tq = Tq;
  a.Tk = Tk;
  a.G = Hq / Hkv;
  a.scale = scale;
  a.scale_log2 = scale * vca::kLog2e;
  a.inv_scale = 1.f / scale;
  a.dq_accumulate = (flags & ATTN_DQ_ACCUMULATE) ? 1 : 0;
  set_ext(a, ext, scale, false);
  return hip_status(bwd_launcher(dtype)(a, Dqk, Dv, causal != 0, num_segments, Hq, Hkv, max_q, Tq,
                                        Tk, tg, workspace, stream),
                    "attn_bwd_varlen launch");
}

int attn_merge(const void* out_a, int dtype_a, const float* lse_a, const void* out_b, int dtype_b,
               const float* lse_b, float* out, float* lse, void* out_copy, int copy_dtype, int rows,
               int H, int Dv, hipStream_t stream) {
  g_last_error.clear();
  if (rows < 0 || H <= 0 || Dv <= 0) return fail(ATTN_E_INVALID, "rows >= 0, H > 0, Dv > 0 required");
  auto known = [](int t) { return t == ATTN_BF16 || t == ATTN_F32 || t == ATTN_F16; };
  if (!known(dtype_a) || !known(dtype_b))
    return fail(ATTN_E_UNSUPPORTED, "merge inputs must be ATTN_BF16, ATTN_F32 or ATTN_F16");
  if (out_copy && copy_dtype != ATTN_BF16 && copy_dtype != ATTN_F16)
    return fail(ATTN_E_UNSUPPORTED, "the merge's copy must be ATTN_BF16 or ATTN_F16");
  if (rows == 0) return ok();
  if (!out_a || !out_b || !lse_a || !lse_b || !out || !lse)
    return fail(ATTN_E_INVALID, "merge pointer is NULL");
  vca::MergeArgs a{};
  a.out_a = out_a;
  a.out_b = out_b;
  a.a_type = dtype_a;
  a.b_type = dtype_b;
  a.lse_a = lse_a;
  a.lse_b = lse_b;
  a.out = out;
  a.lse = lse;
  a.out_copy = static_cast<uint16_t*>(out_copy);
  a.copy_type = copy_dtype;
  a.rows = rows;
  a.H = H;
  a.Dv = Dv;
  return hip_status(vca::launch_merge(a, stream), "attn_merge launch");
}

int attn_zero_rows(void* out, int dtype, int64_t ob, int64_t oh, int64_t on, float* lse,
                   int64_t lse_sb, int64_t lse_sh, const uint8_t* rows, int B, int H, int S, int D,
                   hipStream_t stream) {
  g_last_error.clear();
  if (B < 0 || H < 0 || S < 0 || D < 0) return fail(ATTN_E_INVALID, "B, H, S, D >= 0 required");
  if (dtype != ATTN_BF16 && dtype != ATTN_F32 && dtype != ATTN_F16)
    return fail(ATTN_E_UNSUPPORTED, "zero_rows: out must be ATTN_BF16, ATTN_F32 or ATTN_F16");
  if (B == 0 || H == 0 || S == 0) return ok();
  if (!out || !rows) return fail(ATTN_E_INVALID, "zero_rows pointer is NULL");
  vca::ZeroRowsArgs a{};
  a.out = out;
  a.f32 = dtype == ATTN_F32;
  a.ob = ob;
  a.oh = oh;
  a.on = on;
  a.lse = lse;
  a.lse_sb = lse_sb;
  a.lse_sh = lse_sh;
  a.rows = rows;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  return hip_status(vca::launch_zero_rows(a, stream), "attn_zero_rows launch");
}

}  // extern "C"

// ---- packed ring layout: row movement and the in-place live-row merge ----
namespace {

int ring_esz(int dtype) {
  return dtype == ATTN_F32 ? 4 : (dtype == ATTN_BF16 || dtype == ATTN_F16) ? 2 : 0;
}

// Checks of a [B, H, S, D] view moved in 16-byte pieces.
int check_rows_view(const char* name, const void* p, int64_t sb, int64_t sh, int64_t sn, int esz,
                    int D) {
  if (!p) return fail(ATTN_E_INVALID, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(ATTN_E_INVALID, std::string(name) + " is not 16-byte aligned");
  const int64_t per = 16 / esz;
  if (sb < 0 || sh < 0 || sn < 0 || sb % per || sh % per || sn % per)
    return fail(ATTN_E_INVALID, std::string(name) + " strides must be non-negative multiples of " +
                                    std::to_string(per));
  if ((int64_t)D * esz % 16) return fail(ATTN_E_INVALID, "D * element size must be a multiple of 16");
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_gather_rows(int dtype, const void* src, int64_t sb, int64_t sh, int64_t sn,
                     const int32_t* index, int B, int H, int S, int D, int T, void* dst,
                     int dst_dtype, hipStream_t stream) {
  g_last_error.clear();
  const int esz = ring_esz(dtype);
  if (!esz) return fail(ATTN_E_UNSUPPORTED, "dtype must be ATTN_BF16, ATTN_F16 or ATTN_F32");
  const bool convert = dst_dtype != dtype;
  if (convert && !(dtype == ATTN_F32 && (dst_dtype == ATTN_BF16 || dst_dtype == ATTN_F16)))
    return fail(ATTN_E_UNSUPPORTED, "gather converts only fp32 rows to ATTN_BF16 / ATTN_F16");
  if (convert && D % 8) return fail(ATTN_E_INVALID, "converting gather needs D % 8 == 0");
  if (B < 0 || H <= 0 || S < 0 || D <= 0 || T < 0 || (int64_t)T > (int64_t)B * S)
    return fail(ATTN_E_INVALID, "sizes: B, S, T >= 0, H, D > 0, T <= B * S");
  if (T == 0) return ok();
  int st;
  if ((st = check_rows_view("src", src, sb, sh, sn, esz, D))) return st;
  if (!index || !dst || !aligned16(dst)) return fail(ATTN_E_INVALID, "index / dst NULL or dst unaligned");
  vca::RingRowsArgs a{};
  a.dense = const_cast<void*>(src);
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.packed = dst;
  a.index = index;
  a.B = B;
  a.H = H;
  a.S = S;
  a.T = T;
  a.D = D;
  a.type = dtype;
  a.esz = esz;
  a.dst_type = dst_dtype;
  a.mode = convert ? 3 : 0;
  return hip_status(vca::launch_ring_rows(a, vca::kRingRows, stream), "attn_gather_rows launch");
}

int attn_scatter_rows(int dtype, const void* src, const int32_t* index, int T, int H, int D,
                      void* dst, int64_t sb, int64_t sh, int64_t sn, int B, int S, int mode,
                      hipStream_t stream) {
  g_last_error.clear();
  const int esz = ring_esz(dtype);
  if (!esz) return fail(ATTN_E_UNSUPPORTED, "dtype must be ATTN_BF16, ATTN_F16 or ATTN_F32");
  if (mode != ATTN_ROWS_ASSIGN && mode != ATTN_ROWS_ASSIGN_ZERO_REST && mode != ATTN_ROWS_ADD)
    return fail(ATTN_E_INVALID, "unknown scatter mode");
  if (B < 0 || H <= 0 || S < 0 || D <= 0 || T < 0 || (int64_t)T > (int64_t)B * S)
    return fail(ATTN_E_INVALID, "sizes: B, S, T >= 0, H, D > 0, T <= B * S");
  if ((int64_t)B * S == 0) return ok();
  int st;
  if ((st = check_rows_view("dst", dst, sb, sh, sn, esz, D))) return st;
  if (T > 0 && (!index || !src || !aligned16(src)))
    return fail(ATTN_E_INVALID, "index / src NULL or src unaligned");
  vca::RingRowsArgs a{};
  a.dense = dst;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.packed = const_cast<void*>(src);
  a.index = index;
  a.B = B;
  a.H = H;
  a.S = S;
  a.T = T;
  a.D = D;
  a.type = dtype;
  a.esz = esz;
  if (mode == ATTN_ROWS_ASSIGN_ZERO_REST &&
      (st = hip_status(vca::launch_ring_rows(a, vca::kRingFill, stream), "attn_scatter_rows fill")))
    return st;
  a.mode = mode == ATTN_ROWS_ADD ? 2 : 1;
  return hip_status(vca::launch_ring_rows(a, vca::kRingRows, stream), "attn_scatter_rows launch");
}

int attn_gather_lse(const float* lse_dense, const int32_t* index, int B, int H, int S, int T,
                    float* lse_packed, hipStream_t stream) {
  g_last_error.clear();
  if (B < 0 || H <= 0 || S < 0 || T < 0 || (int64_t)T > (int64_t)B * S)
    return fail(ATTN_E_INVALID, "sizes: B, S, T >= 0, H > 0, T <= B * S");
  if (T == 0) return ok();
  if (!lse_dense || !index || !lse_packed) return fail(ATTN_E_INVALID, "pointer is NULL");
  vca::RingRowsArgs a{};
  a.lse_dense = const_cast<float*>(lse_dense);
  a.lse_packed = lse_packed;
  a.index = index;
  a.B = B;
  a.H = H;
  a.S = S;
  a.T = T;
  a.mode = 0;
  return hip_status(vca::launch_ring_rows(a, vca::kRingLse, stream), "attn_gather_lse launch");
}

int attn_scatter_lse(const float* lse_packed, const int32_t* index, int T, int H, float* lse_dense,
                     int B, int S, int fill_rest, hipStream_t stream) {
  g_last_error.clear();
  if (B < 0 || H <= 0 || S < 0 || T < 0 || (int64_t)T > (int64_t)B * S)
    return fail(ATTN_E_INVALID, "sizes: B, S, T >= 0, H > 0, T <= B * S");
  if ((int64_t)B * S == 0) return ok();
  if (!lse_dense || (T > 0 && (!index || !lse_packed)))
    return fail(ATTN_E_INVALID, "pointer is NULL");
  vca::RingRowsArgs a{};
  a.lse_dense = lse_dense;
  a.lse_packed = const_cast<float*>(lse_packed);
  a.index = index;
  a.B = B;
  a.H = H;
  a.S = S;
  a.T = T;
  a.D = 0;
  a.esz = 4;
  int st;
  if (fill_rest &&
      (st = hip_status(vca::launch_ring_rows(a, vca::kRingFill, stream), "attn_scatter_lse fill")))
    return st;
  a.mode = 1;
  return hip_status(vca::launch_ring_rows(a, vca::kRingLse, stream), "attn_scatter_lse launch");
}

int attn_merge_rows(float* out_acc, int64_t sb, int64_t sh, int64_t sn, float* lse_acc, int B,
                    int S, const void* out_b, int dtype_b, const float* lse_b,
                    const int32_t* index, int T, int H, int D, hipStream_t stream) {
  g_last_error.clear();
  const int esz = ring_esz(dtype_b);
  if (!esz) return fail(ATTN_E_UNSUPPORTED, "dtype_b must be ATTN_BF16, ATTN_F16 or ATTN_F32");
  if (B < 0 || H <= 0 || S < 0 || D <= 0 || T < 0 || (int64_t)T > (int64_t)B * S)
    return fail(ATTN_E_INVALID, "sizes: B, S, T >= 0, H, D > 0, T <= B * S");
  if (T == 0) return ok();
  if (!out_acc || !lse_acc || !out_b || !lse_b || !index)
    return fail(ATTN_E_INVALID, "merge_rows pointer is NULL");
  if (sb < 0 || sh < 0 || sn < 0) return fail(ATTN_E_INVALID, "strides must be non-negative");
  vca::RingRowsArgs a{};
  a.dense = out_acc;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.packed = const_cast<void*>(out_b);
  a.lse_dense = lse_acc;
  a.lse_packed = const_cast<float*>(lse_b);
  a.index = index;
  a.B = B;
  a.H = H;
  a.S = S;
  a.T = T;
  a.D = D;
  a.type = dtype_b;
  a.esz = esz;
  return hip_status(vca::launch_ring_rows(a, vca::kRingMerge, stream), "attn_merge_rows launch");
}

}  // extern "C"


