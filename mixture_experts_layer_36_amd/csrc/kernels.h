// Launch interface of libmoe's bandwidth / routing kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kDispatchBlock = 256;  // tokens per block of the stable-rank kernels

struct RouteArgs {
  const void* x; const void* w; uint32_t* wpack;  // wpack: workspace, bf16 weights in MFMA operand order
  const float* bias;
  float* logits; int32_t* topk_idx; float* topk_w;
  int64_t T; int d; int E; int k; int gating;
};

struct DispatchArgs {
  const void* x; const int32_t* topk_idx;
  void* x_perm; int32_t* row_of; int32_t* assign_of_row;
  int32_t* raw_counts; int32_t* expert_counts; int64_t* expert_offsets;
  int32_t* send_counts; int64_t* send_offsets;
  // workspace
  int32_t* block_counts; int32_t* block_base; int64_t* expert_start;  // the last two: many blocks only
  int64_t T; int64_t d; int E; int k; int64_t C; int R; int placement;
};

// Token chunks [t[r], t[r + 1]) for r < chunks, t[0] = 0, t[chunks] = T.
constexpr int kMaxChunks = 16;
struct ChunkBounds {
  int64_t t[kMaxChunks + 1];
  int chunks;
};

struct ChunkRowsArgs {
  const int32_t* topk_idx; const int32_t* row_of; const int64_t* expert_offsets;
  int64_t* rows;  // [chunks + 1][E]
  ChunkBounds cb;
  int64_t T; int E; int k; int R; int placement;
};

struct CombineArgs {
  const void* y_perm; const int32_t* row_of; const float* topk_w;
  const void* y_shared; void* y;                 // forward
  const void* dy; void* dy_perm; float* d_topk_w; // backward
  int64_t T; int64_t d; int k;
};

struct RouteBwdArgs {
  const void* x; const float* logits; const int32_t* topk_idx; const float* d_topk_w;
  const float* dlogits_add;  // nullable: another gradient of the logits, added to the gating Jacobian's
  float* dlogits; void* dw_router; float* partial;
  int64_t T; int64_t d; int E; int k; int gating;
};

struct DispatchBwdArgs {
  const void* dx_perm; const int32_t* row_of; const float* dlogits; const void* w_router;
  const void* dx_add; void* dx;
  int64_t T; int64_t d; int E; int k;
};

struct AuxArgs {
  const float* logits; const int32_t* raw_counts; float coef;
  float* loss;       // forward: device scalar
  float* partial;    // forward: workspace, aux_ws_bytes(E)
  float* dlogits;    // backward: [T, E]
  int64_t T; int E; int k;
};

hipError_t launch_route(const RouteArgs& a, bool bf16_dtype, hipStream_t st);
// bytes of ws the bf16 route uses for its re-packed copy of w_router
size_t route_ws_bytes(int64_t d, int64_t E);
hipError_t launch_dispatch(const DispatchArgs& a, bool bf16_dtype, hipStream_t st);  // x_perm null: layout only
hipError_t launch_permute(const DispatchArgs& a, bool bf16_dtype, hipStream_t st);   // the row copy alone
hipError_t launch_chunk_rows(const ChunkRowsArgs& a, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, bool bf16_dtype, hipStream_t st);
hipError_t launch_combine_bwd(const CombineArgs& a, bool bf16_dtype, hipStream_t st);
hipError_t launch_route_bwd(const RouteBwdArgs& a, bool bf16_dtype, hipStream_t st);
hipError_t launch_dispatch_bwd(const DispatchBwdArgs& a, bool bf16_dtype, hipStream_t st);

int router_wgrad_blocks(int64_t T);
// compute units of the current device (asked once per device)
hipError_t device_cus(int* cus);

hipError_t launch_aux_loss(const AuxArgs& a, hipStream_t st);
hipError_t launch_aux_loss_bwd(const AuxArgs& a, hipStream_t st);
// bytes of ws the balance loss uses for its partial sums
size_t aux_ws_bytes(int64_t E);

}  // namespace moe
