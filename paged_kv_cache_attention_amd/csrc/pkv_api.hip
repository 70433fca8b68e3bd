// C ABI of libpkv: argument validation, workspace sizing and kernel dispatch.
// The contract of every entry point is documented in include/pkv.h.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// PKV_DEBUG=1 in the environment turns on the device-side contract check;
// read once, at the first call that could run it.
bool debug_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("PKV_DEBUG");
    return v && v[0] == '1';
  }();
  return on;
}

int elem_bytes(pkv_dtype dt) { return dt == PKV_BF16 ? 2 : 4; }

pkv_status check_dtype(pkv_dtype dt) {
  if (dt != PKV_FP32 && dt != PKV_BF16) return fail(PKV_EINVAL, "unknown dtype %d", (int)dt);
  return PKV_OK;
}

pkv_status check_pool_shape(int Hkv, int D, int block_size, int max_blocks, int N_blocks) {
  if (Hkv < 1 || D < 1 || block_size < 1 || max_blocks < 1 || N_blocks < 1)
    return fail(PKV_EINVAL, "Hkv, D, block_size, max_blocks and N_blocks must be positive");
  if (block_size != 16) return fail(PKV_EUNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
  if (D != 64 && D != 128) return fail(PKV_EUNSUPPORTED, "head dim %d unsupported (64 or 128)", D);
  if ((long long)max_blocks * block_size > (1LL << 30)) return fail(PKV_EINVAL, "max_blocks too large");
  return PKV_OK;
}

// Device flag for the PKV_DEBUG contract check, one per device.
int* debug_flag() {
  static std::mutex mu;
  static int* flags[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!flags[dev] && hipMalloc(reinterpret_cast<void**>(&flags[dev]), sizeof(int)) != hipSuccess) flags[dev] = nullptr;
  return flags[dev];
}

pkv_status debug_validate(const int32_t* tables, const int32_t* lens, int B, int T, int len_add, int block_size,
                          int max_blocks, int N_blocks, hipStream_t s, int* flag = nullptr) {
  if (!flag) flag = debug_flag();
  if (!flag) return fail(PKV_EHIP, "PKV_DEBUG: cannot allocate the check flag");
  pkv_status st = from_hip(hipMemsetAsync(flag, 0, sizeof(int), s), "PKV_DEBUG memset");
  if (st != PKV_OK) return st;
  st = from_hip(pkv::launch_validate(tables, lens, B, T, len_add, block_size, max_blocks, N_blocks, flag, s), "PKV_DEBUG check");
  if (st != PKV_OK) return st;
  int host = 0;
  st = from_hip(hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, s), "PKV_DEBUG copy");
  if (st != PKV_OK) return st;
  st = from_hip(hipStreamSynchronize(s), "PKV_DEBUG sync");
  if (st != PKV_OK) return st;
  if (host) return fail(PKV_EINVAL, "PKV_DEBUG: a context length or a used block-table entry is out of range");
  return PKV_OK;
}

int partitions_max(int max_blocks, int block_size, int partition_size) {
  const long long tokens = (long long)max_blocks * block_size;
  return (int)((tokens + partition_size - 1) / partition_size);
}

}  // namespace

// Scratch of the allocation-free decode entry point: a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never uses the array's name as an address: the device address is
// looked up once per device with hipGetSymbolAddress and kept.  The first
// kScratchHead bytes hold the PKV_DEBUG flag; the decode workspace follows.
constexpr size_t kScratchHead = 256;
static __device__ __align__(256) unsigned char scratch[kScratchHead + PKV_NOALLOC_SCRATCH_BYTES];

static pkv_status noalloc_scratch(unsigned char** base) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned char* addr[kMaxDevices] = {nullptr};
  int dev = 0;
  pkv_status st = from_hip(hipGetDevice(&dev), "hipGetDevice");
  if (st != PKV_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {   // with this device current: its own copy of the array
    void* p = nullptr;
    if ((st = from_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) != PKV_OK)
      return st;
    addr[dev] = static_cast<unsigned char*>(p);
  }
  *base = addr[dev];
  return PKV_OK;
}

// K/V rows, queries and outputs move with 16-byte vector loads and stores.
static bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15)) return false;
  return true;
}
static pkv_status misaligned() { return fail(PKV_EINVAL, "tensor arguments must be 16-byte aligned"); }

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

size_t pkv_decode_workspace_bytes(int B, int T, int Hq, int D, int max_blocks, int block_size, int partition_size) {
  if (B < 0 || T < 1 || Hq < 1 || D < 1 || max_blocks < 1 || block_size < 1 || partition_size < 0) return 0;
  if (partition_size == 0) {
    const size_t a = pkv::stream_workspace_bytes(B, T, Hq, D), b = pkv::verify_workspace_bytes(B, T, Hq, D);
    return a > b ? a : b;
  }
  // the documented partials, then (for the MFMA tile) its plan and piece slots
  const unsigned long long P = (unsigned long long)partitions_max(max_blocks, block_size, partition_size);
  const unsigned long long rows = (unsigned long long)B * T * Hq;
  const size_t partials = (size_t)(rows * P * (unsigned long long)(D + 1) * 4ull);
  return (partials + 255) / 256 * 256 + pkv::verify_partition_extra_bytes(B, T, Hq, D);
}

size_t pkv_prefill_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                   int piece_tokens) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || block_size != 16 || max_blocks < 1 ||
      piece_tokens < 0)
    return 0;
  return pkv::prefill_workspace_bytes(B, T, Hq, Hkv, D, max_blocks, piece_tokens);
}

int pkv_prefill_piece_tokens(int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks) {
  if (block_size != 16 || max_blocks < 1 || (D != 64 && D != 128)) return 0;
  return pkv::prefill_piece_tokens(B, T, Hq, Hkv, D, max_blocks, pkv::device_cus());
}

pkv_status paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens_pre, int B, int T, int Hkv, int D,
                           int block_size, int max_blocks, int N_blocks, pkv_dtype dtype, void* stream) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || T < 1) return fail(PKV_EINVAL, "B must be >= 0 and T >= 1");
  if ((st = check_pool_shape(Hkv, D, block_size, max_blocks, N_blocks)) != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !context_lens_pre)
    return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({k_new, v_new, k_pool, v_pool})) return misaligned();
  if ((long long)B * T > (1LL << 30)) return fail(PKV_EINVAL, "B*T too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The append targets positions lens_pre .. lens_pre+T-1: check them as a context of lens_pre+T.
  if (debug_enabled() &&
      (st = debug_validate(block_tables, context_lens_pre, B, T, T, block_size, max_blocks, N_blocks, s)) != PKV_OK)
    return st;
  return from_hip(pkv::launch_append(k_new, v_new, k_pool, v_pool, block_tables, context_lens_pre, B, T, Hkv, D,
                                     block_size, max_blocks, N_blocks, elem_bytes(dtype), s),
                  "paged_kv_append launch");
}

pkv_status paged_kv_append_rope(void* q, int Hq, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens_pre, int B, int T, int Hkv,
                                int D, int block_size, int max_blocks, int N_blocks, float rope_theta, pkv_dtype dtype,
                                void* stream) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || T < 1) return fail(PKV_EINVAL, "B must be >= 0 and T >= 1");
  if ((st = check_pool_shape(Hkv, D, block_size, max_blocks, N_blocks)) != PKV_OK) return st;
  if (!std::isfinite(rope_theta) || rope_theta <= 0.f) return fail(PKV_EINVAL, "rope_theta must be finite and > 0");
  if (q && (Hq < 1 || Hq % Hkv)) return fail(PKV_EINVAL, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (B == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !context_lens_pre)
    return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({q, k_new, v_new, k_pool, v_pool})) return misaligned();
  if ((long long)B * T > (1LL << 30)) return fail(PKV_EINVAL, "B*T too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled() &&
      (st = debug_validate(block_tables, context_lens_pre, B, T, T, block_size, max_blocks, N_blocks, s)) != PKV_OK)
    return st;
  return from_hip(pkv::launch_append_rope(q, Hq, k_new, v_new, k_pool, v_pool, block_tables, context_lens_pre, B, T,
                                          Hkv, D, block_size, max_blocks, N_blocks, (double)rope_theta,
                                          dtype == PKV_BF16, s),
                  "paged_kv_append_rope launch");
}

pkv_status paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int n, int Hkv,
                                int D, int block_size, int N_blocks, pkv_dtype dtype, void* stream) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (n < 0) return fail(PKV_EINVAL, "n must be >= 0");
  if ((st = check_pool_shape(Hkv, D, block_size, 1, N_blocks)) != PKV_OK) return st;
  if (n == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({k_pool, v_pool})) return misaligned();
  return from_hip(pkv::launch_copy_blocks(k_pool, v_pool, src, dst, n, Hkv, D, block_size, N_blocks, elem_bytes(dtype),
                                          static_cast<hipStream_t>(stream)),
                  "paged_kv_copy_blocks launch");
}

pkv_status paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                           const int32_t* context_lens, void* k_out, void* v_out, int B, int max_len, int Hkv, int D,
                           int block_size, int max_blocks, int N_blocks, pkv_dtype dtype, void* stream) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || max_len < 0) return fail(PKV_EINVAL, "B and max_len must be >= 0");
  if ((st = check_pool_shape(Hkv, D, block_size, max_blocks, N_blocks)) != PKV_OK) return st;
  if (B == 0 || max_len == 0) return PKV_OK;
  if (!k_pool || !v_pool || !block_tables || !context_lens || !k_out || !v_out)
    return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({k_pool, v_pool, k_out, v_out})) return misaligned();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled() && (st = debug_validate(block_tables, context_lens, B, 0, 0, block_size, max_blocks, N_blocks, s)) !=
                             PKV_OK)
    return st;
  return from_hip(pkv::launch_gather(k_pool, v_pool, block_tables, context_lens, k_out, v_out, B, max_len, Hkv, D,
                                     block_size, max_blocks, N_blocks, elem_bytes(dtype), s),
                  "paged_kv_gather launch");
}

}  // extern "C"

// The decode entry points' common body.  noalloc: the workspace and the
// PKV_DEBUG flag live in the library's static device scratch (its size is
// checked before anything runs, and nothing is allocated).
static pkv_status decode_impl(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                              const int32_t* context_lens, void* out, float* lse_out, int B, int T, int Hq, int Hkv,
                              int D, int block_size, int max_blocks, int N_blocks, float scale, int partition_size,
                              void* workspace, size_t workspace_bytes, pkv_dtype dtype, void* stream, bool noalloc) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || T < 1 || Hq < 1) return fail(PKV_EINVAL, "B must be >= 0, T and Hq >= 1");
  if ((st = check_pool_shape(Hkv, D, block_size, max_blocks, N_blocks)) != PKV_OK) return st;
  if (Hq % Hkv) return fail(PKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "Hq/Hkv = %d unsupported", G);
  if (Hq % 4) return fail(PKV_EUNSUPPORTED, "Hq must be a multiple of 4");
  if (T > 16) return fail(PKV_EUNSUPPORTED, "T = %d unsupported (at most 16 query tokens)", T);
  if (dtype == PKV_FP32 && D == 128 && G == 1)
    return fail(PKV_EUNSUPPORTED, "fp32 with D=128 needs Hq/Hkv >= 2");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (partition_size < 0 || partition_size % block_size)
    return fail(PKV_EINVAL, "partition_size must be 0 or a positive multiple of block_size");
  if (B == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({q, k_pool, v_pool, out})) return misaligned();
  if (out == q || out == k_pool || out == v_pool) return fail(PKV_EINVAL, "out must not alias an input");

  pkv::DecodeArgs a{};
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool; a.block_tables = block_tables; a.context_lens = context_lens;
  a.out = out; a.lse_out = lse_out;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.block_size = block_size; a.max_blocks = max_blocks;
  a.N_blocks = N_blocks; a.scale = scale; a.bf16 = dtype == PKV_BF16;
  const size_t need = pkv_decode_workspace_bytes(B, T, Hq, D, max_blocks, block_size, partition_size);
  int* dbg_flag = nullptr;
  if (noalloc) {
    if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
      return fail(PKV_EWORKSPACE,
                  "these sizes need %zu bytes of scratch; the allocation-free entry point has %zu (use "
                  "paged_attention_decode with a workspace)",
                  need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    unsigned char* base = nullptr;
    if ((st = noalloc_scratch(&base)) != PKV_OK) return st;
    dbg_flag = reinterpret_cast<int*>(base);
    workspace = base + kScratchHead;
    workspace_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  }
  if (need && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled() && (st = debug_validate(block_tables, context_lens, B, T, 0, block_size, max_blocks, N_blocks, s,
                                              dbg_flag)) != PKV_OK)
    return st;
  const bool fixed_split = partition_size > 0 && partition_size < max_blocks * block_size;
  if (partition_size == 0 && pkv::verify_tile_for(a))
    return from_hip(pkv::launch_verify_mfma(a, workspace, s), "paged_attention_decode verify launch");
  if (partition_size > 0 && pkv::verify_tile_for(a)) {   // split-KV partitions on the MFMA tile
    a.part_tokens = partition_size;
    a.P_max = partitions_max(max_blocks, block_size, partition_size);
    return from_hip(pkv::launch_verify_mfma(a, workspace, s), "paged_attention_decode partition launch");
  }
  if (partition_size == 0 && pkv::stream_supported(a))
    return from_hip(pkv::launch_decode_stream(a, workspace, s), "paged_attention_decode launch");
  if (fixed_split) {
    a.part_tokens = partition_size;
    a.P_max = partitions_max(max_blocks, block_size, partition_size);
    a.part_out = static_cast<float*>(workspace);
    a.part_lse = a.part_out + (size_t)B * T * Hq * a.P_max * D;
  } else {
    a.part_tokens = max_blocks * block_size;
    a.P_max = 1;
  }
  if ((unsigned long long)a.P_max * T * (Hq / 4) * B > (1ull << 31) - 256)
    return fail(PKV_EINVAL, "too many work items");
  st = from_hip(pkv::launch_decode_valu(a, s), "paged_attention_decode launch");
  if (st != PKV_OK || !fixed_split) return st;
  return from_hip(pkv::launch_lse_reduce(a.part_out, a.part_lse, out, lse_out, B, T, Hq, D, a.P_max, a.bf16,
                                         context_lens, partition_size, s),
                  "lse_reduce launch");
}


extern "C" {

pkv_status paged_attention_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, void* out, float* lse_out, int B, int T, int Hq, int Hkv,
                                  int D, int block_size, int max_blocks, int N_blocks, float scale, int partition_size,
                                  void* workspace, size_t workspace_bytes, pkv_dtype dtype, void* stream) {
  return decode_impl(q, k_pool, v_pool, block_tables, context_lens, out, lse_out, B, T, Hq, Hkv, D, block_size,
                     max_blocks, N_blocks, scale, partition_size, workspace, workspace_bytes, dtype, stream, false);
}

pkv_status paged_attention_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* block_tables, const int32_t* context_lens, void* out,
                                          float* lse_out, int B, int T, int Hq, int Hkv, int D, int block_size,
                                          int max_blocks, int N_blocks, float scale, int partition_size,
                                          pkv_dtype dtype, void* stream) {
  return decode_impl(q, k_pool, v_pool, block_tables, context_lens, out, lse_out, B, T, Hq, Hkv, D, block_size,
                     max_blocks, N_blocks, scale, partition_size, nullptr, 0, dtype, stream, true);
}

pkv_status paged_attention_prefill(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                   const int32_t* context_lens, void* out, float* lse_out, int B, int T, int Hq, int Hkv,
                                   int D, int block_size, int max_blocks, int N_blocks, float scale, int piece_tokens,
                                   void* workspace, size_t workspace_bytes, pkv_dtype dtype, void* stream) {
  pkv_status st = check_dtype(dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || T < 1 || Hq < 1) return fail(PKV_EINVAL, "B must be >= 0, T and Hq >= 1");
  if ((st = check_pool_shape(Hkv, D, block_size, max_blocks, N_blocks)) != PKV_OK) return st;
  if (Hq % Hkv) return fail(PKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "Hq/Hkv = %d unsupported", G);
  if (dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "paged_attention_prefill computes in bf16 only");
  if (T > pkv::kPrefillMaxT) return fail(PKV_EUNSUPPORTED, "T = %d unsupported (at most %d)", T, pkv::kPrefillMaxT);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (piece_tokens < 0 || piece_tokens % pkv::kPrefillStep)
    return fail(PKV_EINVAL, "piece_tokens (%d) must be 0 or a positive multiple of %d", piece_tokens,
                pkv::kPrefillStep);
  if (B == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return fail(PKV_EINVAL, "null pointer argument");
  if (!all_aligned16({q, k_pool, v_pool, out})) return misaligned();
  if (out == q || out == k_pool || out == v_pool) return fail(PKV_EINVAL, "out must not alias an input");
  if ((long long)B * T * Hq > (1LL << 30)) return fail(PKV_EINVAL, "B*T*Hq too large");
  const size_t need = pkv::prefill_workspace_bytes(B, T, Hq, Hkv, D, max_blocks, piece_tokens);
  if (need && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (need && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PKV_EINVAL, "workspace must be 16-byte aligned");

  pkv::DecodeArgs a{};
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool; a.block_tables = block_tables; a.context_lens = context_lens;
  a.out = out; a.lse_out = lse_out;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.block_size = block_size; a.max_blocks = max_blocks;
  a.N_blocks = N_blocks; a.scale = scale; a.bf16 = true;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_enabled() && (st = debug_validate(block_tables, context_lens, B, T, 0, block_size, max_blocks, N_blocks, s)) !=
                             PKV_OK)
    return st;
  return from_hip(pkv::launch_prefill(a, need ? piece_tokens : 0, static_cast<float*>(workspace), s),
                  "paged_attention_prefill launch");
}

pkv_status lse_reduce(const float* part_out, const float* part_lse, void* out, float* lse_out, int B, int T, int Hq,
                      int D, int P_max, pkv_dtype out_dtype, void* stream) {
  pkv_status st = check_dtype(out_dtype);
  if (st != PKV_OK) return st;
  if (B < 0 || T < 1 || Hq < 1 || P_max < 1) return fail(PKV_EINVAL, "B must be >= 0; T, Hq and P_max >= 1");
  if (D != 64 && D != 128) return fail(PKV_EUNSUPPORTED, "head dim %d unsupported (64 or 128)", D);
  if (B == 0) return PKV_OK;
  if (!part_out || !part_lse || !out) return fail(PKV_EINVAL, "null pointer argument");
  if ((long long)B * T * Hq > (1LL << 30)) return fail(PKV_EINVAL, "too many rows");
  return from_hip(pkv::launch_lse_reduce(part_out, part_lse, out, lse_out, B, T, Hq, D, P_max,
                                         out_dtype == PKV_BF16, nullptr, 0, static_cast<hipStream_t>(stream)),
                  "lse_reduce launch");
}

}  // extern "C"
