// C ABI of libmegamoe.so: host-side argument checks, then kernel launches on the caller's stream.
// Every check runs before the first HIP call, so invalid arguments are reported without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/megamoe.h"
#include "internal.h"

using namespace megamoe;

namespace {

// Per-device cache of "is this gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int32_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MEGAMOE_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return MEGAMOE_OK;
    if (c == 2) return MEGAMOE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MEGAMOE_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MEGAMOE_OK : MEGAMOE_ERR_DEVICE;
}

int32_t launch_status(hipError_t e) { return e == hipSuccess ? MEGAMOE_OK : MEGAMOE_ERR_LAUNCH; }

// Tile classes a GEMM call may contain: route assigns 16-row tiles to experts with at most
// kSmallClassMaxTokens tokens unless block_m_override forces one height for all.
bool classes_of(int32_t block_m_override, int32_t max_rows_per_expert, GemmClasses* c) {
  if (block_m_override != 0 && block_m_override != kBlockMSmall && block_m_override != kBlockMLarge) return false;
  if (max_rows_per_expert < 0) return false;
  if (block_m_override == kBlockMSmall) *c = {true, false};
  else if (block_m_override == kBlockMLarge) *c = {false, true};
  else *c = {true, !(max_rows_per_expert > 0 && max_rows_per_expert <= kSmallClassMaxTokens)};
  return true;
}

bool gemm_shape_ok(int32_t E, int32_t H, int32_t I, int64_t M_cap) {
  return E >= 1 && E <= MEGAMOE_MAX_EXPERTS && H >= 256 && I >= 128 && H % 256 == 0 && I % 128 == 0 &&
         M_cap >= 0 && M_cap < (int64_t)1 << 31;
}

bool router_shape_ok(int32_t T, int32_t Eg, int32_t k) {
  return T >= 0 && Eg >= 1 && Eg <= MEGAMOE_ROUTER_MAX_EXPERTS && k >= 1 && k <= 64 && k <= Eg &&
         (int64_t)T * k < ((int64_t)1 << 31);
}

}  // namespace

extern "C" size_t megamoe_route_workspace_bytes(int32_t T, int32_t k, int32_t num_experts);
extern "C" int64_t megamoe_row_capacity(int32_t T, int32_t k, int32_t num_experts, int32_t pad_multiple);

namespace {

// Checks of moe_route_permute's arguments other than the workspace (also made by
// moe_route_logits, moe_route_quantize and moe_route_permute_noalloc).
int32_t route_args_ok_no_ws(int32_t T, int32_t k, int32_t expert_begin, int32_t num_experts, int32_t pad_multiple,
                            int32_t block_m_override, const int32_t* topk_ids, const int32_t* counts,
                            const int32_t* expert_offsets, const int32_t* padded_offsets, const int32_t* row_token,
                            const int32_t* token_rows, const int32_t* sched) {
  if (T < 0 || k < 1 || k > 64 || num_experts < 1 || num_experts > MEGAMOE_MAX_EXPERTS || pad_multiple < 1 ||
      expert_begin < 0)
    return MEGAMOE_ERR_SHAPE;
  if (block_m_override != 0 && block_m_override != kBlockMSmall && block_m_override != kBlockMLarge)
    return MEGAMOE_ERR_SHAPE;
  const int64_t n = (int64_t)T * k;
  const int64_t M_cap = megamoe_row_capacity(T, k, num_experts, pad_multiple);
  if (n >= ((int64_t)1 << 31) || M_cap >= ((int64_t)1 << 31)) return MEGAMOE_ERR_SHAPE;
  if (!counts || !expert_offsets || !padded_offsets || !sched) return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && !row_token) return MEGAMOE_ERR_NULL;
  if (n > 0 && (!topk_ids || !token_rows)) return MEGAMOE_ERR_NULL;
  return MEGAMOE_OK;
}

// All of moe_route_permute's checks, the workspace included.
int32_t route_args_ok(int32_t T, int32_t k, int32_t expert_begin, int32_t num_experts, int32_t pad_multiple,
                      int32_t block_m_override, const int32_t* topk_ids, const int32_t* counts,
                      const int32_t* expert_offsets, const int32_t* padded_offsets, const int32_t* row_token,
                      const int32_t* token_rows, const int32_t* sched, const void* workspace,
                      size_t workspace_bytes) {
  const int32_t rc = route_args_ok_no_ws(T, k, expert_begin, num_experts, pad_multiple, block_m_override, topk_ids,
                                         counts, expert_offsets, padded_offsets, row_token, token_rows, sched);
  if (rc != MEGAMOE_OK) return rc;
  const size_t need = megamoe_route_workspace_bytes(T, k, num_experts);
  if (workspace_bytes < need) return MEGAMOE_ERR_WORKSPACE;
  if (need > 0 && !workspace) return MEGAMOE_ERR_NULL;
  return MEGAMOE_OK;
}

}  // namespace

extern "C" {

int64_t megamoe_row_capacity(int32_t T, int32_t k, int32_t num_experts, int32_t pad_multiple) {
  if (T < 0 || k < 1 || num_experts < 1 || pad_multiple < 1) return -1;
  return (int64_t)T * k + (int64_t)num_experts * (pad_multiple - 1);
}

int64_t megamoe_sched_len(int32_t num_experts) {
  if (num_experts < 1 || num_experts > MEGAMOE_MAX_EXPERTS) return -1;
  return sched_len(num_experts);
}

size_t megamoe_route_workspace_bytes(int32_t T, int32_t k, int32_t num_experts) {
  if (T < 0 || k < 1 || num_experts < 1) return 0;
  const int64_t n = (int64_t)T * k;
  const int64_t nchunks = (n + kRouteChunk - 1) / kRouteChunk;
  return (size_t)(nchunks * num_experts * (int64_t)sizeof(int32_t));
}

size_t megamoe_quant_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return (size_t)quant_amax_parts(rows, cols) * sizeof(float);
}

int32_t moe_router_topk(const float* logits, int32_t T, int32_t num_experts_global, int32_t k, int32_t* topk_ids,
                        float* topk_weights, void* stream) {
  if (!router_shape_ok(T, num_experts_global, k)) return MEGAMOE_ERR_SHAPE;
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_router(logits, T, num_experts_global, k, topk_ids, topk_weights,
                                     static_cast<hipStream_t>(stream)));
}

int32_t moe_route_logits(const float* logits, int32_t T, int32_t num_experts_global, int32_t k, int32_t expert_begin,
                         int32_t num_experts, int32_t pad_multiple, int32_t block_m_override, int32_t* topk_ids,
                         float* topk_weights, int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                         int32_t* row_token, int32_t* token_rows, int32_t* sched, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!router_shape_ok(T, num_experts_global, k)) return MEGAMOE_ERR_SHAPE;
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MEGAMOE_ERR_NULL;
  const int32_t rc = route_args_ok(T, k, expert_begin, num_experts, pad_multiple, block_m_override, topk_ids, counts,
                                   expert_offsets, padded_offsets, row_token, token_rows, sched, workspace,
                                   workspace_bytes);
  if (rc != MEGAMOE_OK) return rc;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t r = launch_status(launch_router(logits, T, num_experts_global, k, topk_ids, topk_weights, s));
  if (r != MEGAMOE_OK) return r;
  return launch_status(launch_route(topk_ids, T, k, expert_begin, num_experts, pad_multiple, block_m_override, counts,
                                    expert_offsets, padded_offsets, row_token,
                                    megamoe_row_capacity(T, k, num_experts, pad_multiple), token_rows, sched,
                                    static_cast<int32_t*>(workspace), s));
}

int32_t moe_route_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin, int32_t num_experts,
                          int32_t pad_multiple, int32_t block_m_override, int32_t* counts, int32_t* expert_offsets,
                          int32_t* padded_offsets, int32_t* row_token, int32_t* token_rows, int32_t* sched,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t rc = route_args_ok(T, k, expert_begin, num_experts, pad_multiple, block_m_override, topk_ids, counts,
                                   expert_offsets, padded_offsets, row_token, token_rows, sched, workspace,
                                   workspace_bytes);
  if (rc != MEGAMOE_OK) return rc;
  const int64_t M_cap = megamoe_row_capacity(T, k, num_experts, pad_multiple);
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_route(topk_ids, T, k, expert_begin, num_experts, pad_multiple, block_m_override, counts,
                                    expert_offsets, padded_offsets, row_token, M_cap, token_rows, sched,
                                    static_cast<int32_t*>(workspace), static_cast<hipStream_t>(stream)));
}

int32_t moe_route_permute_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin,
                                  int32_t num_experts, int32_t pad_multiple, int32_t block_m_override,
                                  int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                                  int32_t* row_token, int32_t* token_rows, int32_t* sched, void* stream) {
  const int32_t rc = route_args_ok_no_ws(T, k, expert_begin, num_experts, pad_multiple, block_m_override, topk_ids,
                                         counts, expert_offsets, padded_offsets, row_token, token_rows, sched);
  if (rc != MEGAMOE_OK) return rc;
  if (megamoe_route_workspace_bytes(T, k, num_experts) > (size_t)MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES)
    return MEGAMOE_ERR_WORKSPACE;
  const int64_t M_cap = megamoe_row_capacity(T, k, num_experts, pad_multiple);
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  int32_t* scratch = nullptr;
  if (route_noalloc_scratch(&scratch) != hipSuccess) return MEGAMOE_ERR_LAUNCH;
  return launch_status(launch_route(topk_ids, T, k, expert_begin, num_experts, pad_multiple, block_m_override, counts,
                                    expert_offsets, padded_offsets, row_token, M_cap, token_rows, sched, scratch,
                                    static_cast<hipStream_t>(stream)));
}

int32_t moe_route_quantize(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin, int32_t num_experts,
                           int32_t pad_multiple, int32_t block_m_override, int32_t* counts, int32_t* expert_offsets,
                           int32_t* padded_offsets, int32_t* row_token, int32_t* token_rows, int32_t* sched,
                           void* route_workspace, size_t route_workspace_bytes, const void* x_bf16, int64_t H,
                           const float* x_gs_in, uint8_t* x_codes, uint8_t* x_scales, float* x_global_scale,
                           void* quant_workspace, size_t quant_workspace_bytes, void* stream) {
  const int32_t rc = route_args_ok(T, k, expert_begin, num_experts, pad_multiple, block_m_override, topk_ids, counts,
                                   expert_offsets, padded_offsets, row_token, token_rows, sched, route_workspace,
                                   route_workspace_bytes);
  if (rc != MEGAMOE_OK) return rc;
  if (H <= 0 || H % 32 != 0 || (int64_t)T > ((int64_t)1 << 40) / H) return MEGAMOE_ERR_SHAPE;
  if (!x_gs_in && !x_global_scale) return MEGAMOE_ERR_NULL;
  if (T > 0 && (!x_bf16 || !x_codes || !x_scales)) return MEGAMOE_ERR_NULL;
  const size_t qneed = x_gs_in ? 0 : megamoe_quant_workspace_bytes(T, H);
  if (quant_workspace_bytes < qneed) return MEGAMOE_ERR_WORKSPACE;
  if (qneed > 0 && !quant_workspace) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t M_cap = megamoe_row_capacity(T, k, num_experts, pad_multiple);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  if (route_quant_fusable(T, k, H))
    return launch_status(launch_route_quant_small(topk_ids, T, k, expert_begin, num_experts, pad_multiple,
                                                  block_m_override, counts, expert_offsets, padded_offsets, row_token,
                                                  M_cap, token_rows, sched, x, H, x_codes, x_scales, x_global_scale,
                                                  x_gs_in, s));
  const int32_t r = launch_status(launch_route(topk_ids, T, k, expert_begin, num_experts, pad_multiple,
                                               block_m_override, counts, expert_offsets, padded_offsets, row_token,
                                               M_cap, token_rows, sched, static_cast<int32_t*>(route_workspace), s));
  if (r != MEGAMOE_OK) return r;
  if (x_gs_in) return launch_status(launch_quant_gs(x, T, H, nullptr, x_gs_in, x_codes, x_scales, s));
  return launch_status(launch_quant(x, T, H, nullptr, nullptr, 0, x_codes, x_scales, x_global_scale,
                                    static_cast<float*>(quant_workspace), s));
}

int32_t nvfp4_quantize_act(const void* x_bf16, int64_t rows, int64_t cols, const int32_t* row_valid,
                           const float* amax_in, int32_t amax_in_count, uint8_t* codes, uint8_t* scales,
                           float* global_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || rows > ((int64_t)1 << 40) / cols) return MEGAMOE_ERR_SHAPE;
  if (amax_in && (amax_in_count < 1 || amax_in_count > 65536)) return MEGAMOE_ERR_SHAPE;
  if (!global_scale) return MEGAMOE_ERR_NULL;
  if (rows > 0 && (!x_bf16 || !codes || !scales)) return MEGAMOE_ERR_NULL;
  const size_t need = amax_in ? 0 : megamoe_quant_workspace_bytes(rows, cols);
  if (workspace_bytes < need) return MEGAMOE_ERR_WORKSPACE;
  if (need > 0 && !workspace) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_quant(static_cast<const uint16_t*>(x_bf16), rows, cols, row_valid, amax_in, amax_in_count, codes, scales,
                                    global_scale, static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_quantize_act_gs(const void* x_bf16, int64_t rows, int64_t cols, const int32_t* row_valid,
                              const float* global_scale_in, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || rows > ((int64_t)1 << 40) / cols) return MEGAMOE_ERR_SHAPE;
  if (!global_scale_in) return MEGAMOE_ERR_NULL;
  if (rows > 0 && (!x_bf16 || !codes || !scales)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_quant_gs(static_cast<const uint16_t*>(x_bf16), rows, cols, row_valid, global_scale_in,
                                       codes, scales, static_cast<hipStream_t>(stream)));
}

// The three grouped GEMMs, with the packed weight codes (nvfp4_pack_weight_codes) or without.
static int32_t gemm_l1(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, const int32_t* row_token,
                       const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                       const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                       const uint8_t* w13_packed, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                       int32_t block_m_override, int32_t max_rows_per_expert, void* h_bf16, float* h_amax_parts,
                       void* stream) {
  GemmClasses cls;
  if (!gemm_shape_ok(E, H, I, M_cap) || !classes_of(block_m_override, max_rows_per_expert, &cls))
    return MEGAMOE_ERR_SHAPE;
  if (!x_gs || !padded_offsets || !counts || !sched || !w13_codes || !w13_scales || !w13_gs || !h_amax_parts)
    return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && (!x_codes || !x_scales || !row_token || !h_bf16)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  if (M_cap == 0)  // no rows: only the amax slots, all 0
    return launch_status(launch_fill_f32(h_amax_parts, MEGAMOE_L1_AMAX_PARTS, 0.0f, static_cast<hipStream_t>(stream)));
  GemmArgs a{x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
             E, H, I, h_bf16, h_amax_parts, 0};
  a.w_packed = w13_packed;
  return launch_status(launch_gemm_l1(a, cls, static_cast<hipStream_t>(stream)));
}

static int32_t gemm_l1_nvfp4(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                             const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                             const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                             const float* w13_gs, const uint8_t* w13_packed, int32_t E, int32_t H, int32_t I,
                             int64_t M_cap, int32_t block_m_override, int32_t max_rows_per_expert, const float* h_gs,
                             uint8_t* h_codes, uint8_t* h_scales, float* h_amax_parts, void* stream) {
  GemmClasses cls;
  if (!gemm_shape_ok(E, H, I, M_cap) || !classes_of(block_m_override, max_rows_per_expert, &cls))
    return MEGAMOE_ERR_SHAPE;
  if (!x_gs || !padded_offsets || !counts || !sched || !w13_codes || !w13_scales || !w13_gs || !h_gs ||
      !h_amax_parts)
    return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && (!x_codes || !x_scales || !row_token || !h_codes || !h_scales)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  if (M_cap == 0)  // no rows: only the amax slots, all 0
    return launch_status(launch_fill_f32(h_amax_parts, MEGAMOE_L1_AMAX_PARTS, 0.0f, static_cast<hipStream_t>(stream)));
  GemmArgs a{x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
             E, H, I, nullptr, h_amax_parts, 0};
  a.q_gs = h_gs;
  a.q_codes = h_codes;
  a.q_scales = h_scales;
  a.w_packed = w13_packed;
  return launch_status(launch_gemm_l1(a, cls, static_cast<hipStream_t>(stream)));
}

static int32_t gemm_l2(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs,
                       const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                       const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs, const uint8_t* w2_packed,
                       int32_t E, int32_t H, int32_t I, int64_t M_cap, int32_t block_m_override,
                       int32_t max_rows_per_expert, void* y_bf16, void* stream) {
  GemmClasses cls;
  if (!gemm_shape_ok(E, H, I, M_cap) || !classes_of(block_m_override, max_rows_per_expert, &cls))
    return MEGAMOE_ERR_SHAPE;
  if (!h_gs || !padded_offsets || !counts || !sched || !w2_codes || !w2_scales || !w2_gs) return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && (!h_codes || !h_scales || !y_bf16)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  if (M_cap == 0) return MEGAMOE_OK;  // no rows: nothing to compute or write
  GemmArgs a{h_codes, h_scales, h_gs, nullptr, padded_offsets, counts, sched, w2_codes, w2_scales, w2_gs,
             E, I, H, y_bf16, nullptr, 0};
  a.w_packed = w2_packed;
  return launch_status(launch_gemm_l2(a, cls, static_cast<hipStream_t>(stream)));
}

int32_t moe_grouped_gemm_l1_silu(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                 const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                                 const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                 const float* w13_gs, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                                 int32_t block_m_override, int32_t max_rows_per_expert, void* h_bf16,
                                 float* h_amax_parts, void* stream) {
  return gemm_l1(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
                 nullptr, E, H, I, M_cap, block_m_override, max_rows_per_expert, h_bf16, h_amax_parts, stream);
}

int32_t moe_grouped_gemm_l1_silu_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                        const int32_t* row_token, const int32_t* padded_offsets,
                                        const int32_t* counts, const int32_t* sched, const uint8_t* w13_codes,
                                        const uint8_t* w13_scales, const float* w13_gs, const uint8_t* w13_packed,
                                        int32_t E, int32_t H, int32_t I, int64_t M_cap, int32_t block_m_override,
                                        int32_t max_rows_per_expert, void* h_bf16, float* h_amax_parts,
                                        void* stream) {
  if (!w13_packed) return MEGAMOE_ERR_NULL;  // K = H is a multiple of 256 for every accepted shape
  return gemm_l1(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
                 w13_packed, E, H, I, M_cap, block_m_override, max_rows_per_expert, h_bf16, h_amax_parts, stream);
}

int32_t moe_grouped_gemm_l1_silu_nvfp4(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                       const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                                       const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                       const float* w13_gs, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                                       int32_t block_m_override, int32_t max_rows_per_expert, const float* h_gs,
                                       uint8_t* h_codes, uint8_t* h_scales, float* h_amax_parts, void* stream) {
  return gemm_l1_nvfp4(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales,
                       w13_gs, nullptr, E, H, I, M_cap, block_m_override, max_rows_per_expert, h_gs, h_codes,
                       h_scales, h_amax_parts, stream);
}

int32_t moe_grouped_gemm_l1_silu_nvfp4_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                              const int32_t* row_token, const int32_t* padded_offsets,
                                              const int32_t* counts, const int32_t* sched, const uint8_t* w13_codes,
                                              const uint8_t* w13_scales, const float* w13_gs,
                                              const uint8_t* w13_packed, int32_t E, int32_t H, int32_t I,
                                              int64_t M_cap, int32_t block_m_override, int32_t max_rows_per_expert,
                                              const float* h_gs, uint8_t* h_codes, uint8_t* h_scales,
                                              float* h_amax_parts, void* stream) {
  if (!w13_packed) return MEGAMOE_ERR_NULL;
  return gemm_l1_nvfp4(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales,
                       w13_gs, w13_packed, E, H, I, M_cap, block_m_override, max_rows_per_expert, h_gs, h_codes,
                       h_scales, h_amax_parts, stream);
}

int32_t moe_grouped_gemm_l2(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs,
                            const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                            const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs, int32_t E, int32_t H,
                            int32_t I, int64_t M_cap, int32_t block_m_override, int32_t max_rows_per_expert,
                            void* y_bf16, void* stream) {
  return gemm_l2(h_codes, h_scales, h_gs, padded_offsets, counts, sched, w2_codes, w2_scales, w2_gs, nullptr, E, H, I,
                 M_cap, block_m_override, max_rows_per_expert, y_bf16, stream);
}

int32_t moe_grouped_gemm_l2_packed(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs,
                                   const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                                   const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                                   const uint8_t* w2_packed, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                                   int32_t block_m_override, int32_t max_rows_per_expert, void* y_bf16,
                                   void* stream) {
  if (I % 256 != 0) return MEGAMOE_ERR_SHAPE;  // the packed layout is in 256-element chunks of K = I
  if (!w2_packed) return MEGAMOE_ERR_NULL;
  return gemm_l2(h_codes, h_scales, h_gs, padded_offsets, counts, sched, w2_codes, w2_scales, w2_gs, w2_packed, E, H,
                 I, M_cap, block_m_override, max_rows_per_expert, y_bf16, stream);
}

int32_t nvfp4_pack_weight_codes(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed, void* stream) {
  if (rows < 16 || rows % 16 != 0 || K < 256 || K % 256 != 0) return MEGAMOE_ERR_SHAPE;
  if (!codes || !packed) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_pack_codes16(codes, rows, K, packed, static_cast<hipStream_t>(stream)));
}

int32_t moe_combine(const void* y_bf16, const int32_t* token_rows, const float* topk_weights, int32_t T, int32_t k,
                    int32_t H, void* out_bf16, void* stream) {
  if (T < 0 || k < 1 || k > 64 || H < 8 || H % 8 != 0) return MEGAMOE_ERR_SHAPE;
  if (T > 0 && (!y_bf16 || !token_rows || !topk_weights || !out_bf16)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_combine(static_cast<const uint16_t*>(y_bf16), token_rows, topk_weights, T, k, H, nullptr,
                                      static_cast<uint16_t*>(out_bf16), static_cast<hipStream_t>(stream)));
}

int32_t moe_combine_shared(const void* y_bf16, const int32_t* token_rows, const float* topk_weights, int32_t T,
                           int32_t k, int32_t H, const void* y_shared_bf16, void* out_bf16, void* stream) {
  if (T < 0 || k < 1 || k > 64 || H < 8 || H % 8 != 0) return MEGAMOE_ERR_SHAPE;
  if (T > 0 && (!y_bf16 || !token_rows || !topk_weights || !y_shared_bf16 || !out_bf16)) return MEGAMOE_ERR_NULL;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  return launch_status(launch_combine(static_cast<const uint16_t*>(y_bf16), token_rows, topk_weights, T, k, H,
                                      static_cast<const uint16_t*>(y_shared_bf16), static_cast<uint16_t*>(out_bf16),
                                      static_cast<hipStream_t>(stream)));
}

size_t megamoe_ffn_sync_bytes(int32_t num_experts) {
  if (num_experts < 1 || num_experts > MEGAMOE_MAX_EXPERTS) return 0;
  return (size_t)(kFfnSyncHeader + (int64_t)num_experts * kFfnSyncStride) * sizeof(uint32_t);
}

static int32_t ffn_fused(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                         const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                         const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                         const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                         const uint8_t* w13_packed, const uint8_t* w2_packed, int32_t E, int32_t H, int32_t I,
                         int64_t M_cap, const float* h_gs_in, void* h_bf16, float* h_amax_parts, uint8_t* h_codes,
                         uint8_t* h_scales, float* h_gs_out, void* y_bf16, void* sync, size_t sync_bytes,
                         void* stream) {
  if (!gemm_shape_ok(E, H, I, M_cap)) return MEGAMOE_ERR_SHAPE;
  if (!x_gs || !padded_offsets || !counts || !sched || !w13_codes || !w13_scales || !w13_gs || !w2_codes ||
      !w2_scales || !w2_gs || !h_amax_parts || !sync)
    return MEGAMOE_ERR_NULL;
  if (!h_gs_in && !h_gs_out) return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && (!x_codes || !x_scales || !row_token || !h_codes || !h_scales || !y_bf16)) return MEGAMOE_ERR_NULL;
  if (M_cap > 0 && !h_gs_in && !h_bf16) return MEGAMOE_ERR_NULL;
  if (sync_bytes < megamoe_ffn_sync_bytes(E)) return MEGAMOE_ERR_WORKSPACE;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M_cap == 0) {  // no rows: the amax slots (all 0) and, without a calibrated scale, gs_h = 1
    const int32_t r = launch_status(launch_fill_f32(h_amax_parts, MEGAMOE_L1_AMAX_PARTS, 0.0f, s));
    if (r != MEGAMOE_OK || h_gs_in) return r;
    return launch_status(launch_fill_f32(h_gs_out, 1, 1.0f, s));
  }
  FfnArgs a{};
  a.l1 = GemmArgs{x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
                  E, H, I, h_gs_in ? nullptr : h_bf16, h_amax_parts, 0};
  if (h_gs_in) {
    a.l1.q_gs = h_gs_in;
    a.l1.q_codes = h_codes;
    a.l1.q_scales = h_scales;
  }
  a.l2 = GemmArgs{h_codes, h_scales, h_gs_in ? h_gs_in : h_gs_out, nullptr, padded_offsets, counts, sched, w2_codes,
                  w2_scales, w2_gs, E, I, H, y_bf16, nullptr, 0};
  a.l1.w_packed = w13_packed;
  a.l2.w_packed = w2_packed;
  a.sync = static_cast<uint32_t*>(sync);
  a.row_valid = row_token;
  a.M_cap = M_cap;
  a.hq_codes = h_codes;
  a.hq_scales = h_scales;
  a.h_gs = h_gs_out;
  return launch_status(launch_ffn_small(a, s));
}

int32_t moe_grouped_ffn_fused(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                              const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                              const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                              const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales,
                              const float* w2_gs, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                              const float* h_gs_in, void* h_bf16, float* h_amax_parts, uint8_t* h_codes,
                              uint8_t* h_scales, float* h_gs_out, void* y_bf16, void* sync, size_t sync_bytes,
                              void* stream) {
  return ffn_fused(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
                   w2_codes, w2_scales, w2_gs, nullptr, nullptr, E, H, I, M_cap, h_gs_in, h_bf16, h_amax_parts,
                   h_codes, h_scales, h_gs_out, y_bf16, sync, sync_bytes, stream);
}

int32_t moe_grouped_ffn_fused_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                     const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                                     const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                     const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                     const float* w2_gs, const uint8_t* w13_packed, const uint8_t* w2_packed,
                                     int32_t E, int32_t H, int32_t I, int64_t M_cap, const float* h_gs_in,
                                     void* h_bf16, float* h_amax_parts, uint8_t* h_codes, uint8_t* h_scales,
                                     float* h_gs_out, void* y_bf16, void* sync, size_t sync_bytes, void* stream) {
  if (I % 256 != 0) return MEGAMOE_ERR_SHAPE;  // the packed layout is in 256-element chunks of K
  if (!w13_packed || !w2_packed) return MEGAMOE_ERR_NULL;
  return ffn_fused(x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_codes, w13_scales, w13_gs,
                   w2_codes, w2_scales, w2_gs, w13_packed, w2_packed, E, H, I, M_cap, h_gs_in, h_bf16, h_amax_parts,
                   h_codes, h_scales, h_gs_out, y_bf16, sync, sync_bytes, stream);
}

size_t megamoe_dense_workspace_bytes(int64_t M) {
  if (M < 0 || M >= ((int64_t)1 << 31)) return 0;
  return (size_t)(kDenseHeader + M) * sizeof(int32_t);
}

int32_t nvfp4_linear(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs, int64_t M, int32_t K,
                     const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int32_t N, void* out_bf16,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!gemm_shape_ok(1, N, K, M)) return MEGAMOE_ERR_SHAPE;
  if (!a_gs || !w_codes || !w_scales || !w_gs || !workspace) return MEGAMOE_ERR_NULL;
  if (M > 0 && (!a_codes || !a_scales || !out_bf16)) return MEGAMOE_ERR_NULL;
  if (workspace_bytes < (size_t)kDenseHeader * sizeof(int32_t)) return MEGAMOE_ERR_WORKSPACE;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  if (M == 0) return MEGAMOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ws = static_cast<int32_t*>(workspace);
  const int32_t r = launch_status(launch_dense_setup((int32_t)M, ws, false, s));
  if (r != MEGAMOE_OK) return r;
  const GemmClasses cls{M <= kSmallClassMaxTokens, M > kSmallClassMaxTokens};  // exactly the group's class
  GemmArgs ga{a_codes, a_scales, a_gs, nullptr, ws + kDensePoff, ws + kDenseCounts, ws + kDenseSched, w_codes,
              w_scales, w_gs, 1, K, N, out_bf16, nullptr, 0};
  return launch_status(launch_gemm_l2(ga, cls, s));
}

int32_t nvfp4_linear_gate_up_silu(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs, int64_t M,
                                  int32_t K, const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                                  int32_t I, void* h_bf16, float* h_amax_parts, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!gemm_shape_ok(1, K, I, M)) return MEGAMOE_ERR_SHAPE;
  if (!a_gs || !w13_codes || !w13_scales || !w13_gs || !h_amax_parts || !workspace) return MEGAMOE_ERR_NULL;
  if (M > 0 && (!a_codes || !a_scales || !h_bf16)) return MEGAMOE_ERR_NULL;
  if (workspace_bytes < megamoe_dense_workspace_bytes(M)) return MEGAMOE_ERR_WORKSPACE;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ws = static_cast<int32_t*>(workspace);
  const int32_t r = launch_status(launch_dense_setup((int32_t)M, ws, true, s));
  if (r != MEGAMOE_OK) return r;
  const GemmClasses cls{M <= kSmallClassMaxTokens, M > kSmallClassMaxTokens};  // exactly the group's class
  GemmArgs ga{a_codes, a_scales, a_gs, ws + kDenseHeader, ws + kDensePoff, ws + kDenseCounts, ws + kDenseSched,
              w13_codes, w13_scales, w13_gs, 1, K, I, h_bf16, h_amax_parts, 0};
  return launch_status(launch_gemm_l1(ga, cls, s));
}

int32_t nvfp4_linear_gate_up_silu_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                        int64_t M, int32_t K, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                        const float* w13_gs, int32_t I, const float* h_gs, uint8_t* h_codes,
                                        uint8_t* h_scales, float* h_amax_parts, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!gemm_shape_ok(1, K, I, M)) return MEGAMOE_ERR_SHAPE;
  if (!a_gs || !w13_codes || !w13_scales || !w13_gs || !h_gs || !h_amax_parts || !workspace) return MEGAMOE_ERR_NULL;
  if (M > 0 && (!a_codes || !a_scales || !h_codes || !h_scales)) return MEGAMOE_ERR_NULL;
  if (workspace_bytes < megamoe_dense_workspace_bytes(M)) return MEGAMOE_ERR_WORKSPACE;
  const int32_t dev = check_device();
  if (dev != MEGAMOE_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ws = static_cast<int32_t*>(workspace);
  const int32_t r = launch_status(launch_dense_setup((int32_t)M, ws, true, s));
  if (r != MEGAMOE_OK) return r;
  const GemmClasses cls{M <= kSmallClassMaxTokens, M > kSmallClassMaxTokens};  // exactly the group's class
  GemmArgs ga{a_codes, a_scales, a_gs, ws + kDenseHeader, ws + kDensePoff, ws + kDenseCounts, ws + kDenseSched,
              w13_codes, w13_scales, w13_gs, 1, K, I, nullptr, h_amax_parts, 0};
  ga.q_gs = h_gs;
  ga.q_codes = h_codes;
  ga.q_scales = h_scales;
  return launch_status(launch_gemm_l1(ga, cls, s));
}

}  // extern "C"
