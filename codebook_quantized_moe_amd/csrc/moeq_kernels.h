// Host-side launchers of the libmoeq kernels (defined in the .hip files next to this one).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq_device.h"

namespace moeq {

struct SkinnyArgs {
    const uint16_t* act;          // gate|up: x [T, H] (natural); down: inter [T*k, I] (pair-split)
    uint32_t act_bytes;           // size of act in bytes (< 2^31)
    const int32_t* offsets;       // [E + 1]
    const int32_t* sorted_pair;   // [T * k]
    const float* topk_w;          // [T * k] (down only)
    const uint8_t* codes0;        // gate or down codes [E, N, K/2]
    const uint8_t* scales0;       // [E, N, K/32]
    const uint8_t* codes1;        // up codes (gate|up only)
    const uint8_t* scales1;
    const uint8_t* table_id;      // [E]
    void* out;                    // gate|up: inter bf16 [T*k, I]; down: yp fp32 [T*k, H]
    int T, k, E;
    int N;                        // weight rows per expert: I (gate|up) or H (down)
    int K;                        // contraction length: H (gate|up) or I (down)
    int out_ld;                   // row stride of out, in elements
    int32_t* queue;               // prefill: 8 work-queue counters (device, zeroed per launch)
    int act_natural;              // few-rows gate|up: act is x in natural K order, put into
                                  // pair-split order in LDS after staging (else already split)
    TableArgs tables;
};

void launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* wr, int E,
                          float* logits, hipStream_t stream);
void launch_route_topk(const float* logits, int T, int E, int k, bool sigmoid, int32_t* ids,
                       float* w, hipStream_t stream);
void launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_pos, hipStream_t stream);
void launch_route_permute(const float* logits, int T, int E, int k, bool sigmoid, int32_t* ids,
                          float* w, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          hipStream_t stream);
void launch_decode(const SkinnyArgs& a, bool gateup, long tiles, int cus, int shape,
                   hipStream_t stream);
int decode_tile_rows();
// max_groups > 0 caps the workgroups (testing: many items per workgroup)
void launch_prefill(const SkinnyArgs& a, bool gateup, long tiles, int cus, int max_groups,
                    hipStream_t stream);
int prefill_tile_rows();
size_t prefill_split_bytes(int T, int H);
size_t prefill_queue_bytes();
void launch_pair_split_rows(const uint16_t* x, int T, int H, uint16_t* xs, int cus,
                            hipStream_t stream);
void launch_combine(const float* yp, const int32_t* pair_pos, const int32_t* offsets, int T, int k,
                    int E, int H, const float* shared_z, const uint16_t* residual, uint16_t* y,
                    hipStream_t stream);
// the whole decode layer in one cooperative launch (gemm_decode.hip)
struct DecodeLayerArgs {
    SkinnyArgs gu, dn;            // the two projections (routing arrays inside the workspace)
    const float* logits;          // [T, E]
    int sigmoid;                  // gating: 0 softmax, 1 sigmoid
    int32_t* ids;                 // [T*k]
    float* w;                     // [T*k]
    int32_t* offsets;             // [E + 1]
    int32_t* sorted_pair;         // [T*k]
    int32_t* pair_pos;            // [T*k]
    const float* yp;              // [T*k, H] (the down projection's output)
    const uint16_t* residual;     // [T, H] or null
    uint16_t* y;                  // [T, H]
    int* barrier;                 // header: arrivals, failure flag, clock stamps, ready flag
    int T, k, E, H;
};
// returns the grid size, or < 0 when the cooperative launch was refused
int launch_decode_layer(const DecodeLayerArgs& L, int cus, hipStream_t stream);

// encoding and grid fit
struct Table8 {
    float v[8];
};
void launch_quantize(const uint16_t* w, long long rows, int K, int N, const TableArgs& ta,
                     const uint8_t* table_id, uint8_t* codes, uint8_t* scales, double* row_err,
                     hipStream_t stream);
size_t lloyd_workspace_bytes(long long rows);
void launch_lloyd_stats(const uint16_t* w, long long rows, int K, const Table8& tab, float gmax,
                        double* part, int accumulate, double* stats, hipStream_t stream);
void launch_select_arms(const double* err_a, const double* err_b, int E, int N, int accumulate,
                        uint8_t* table_id, double* expert_err, hipStream_t stream);
// shared expert: routing of every token to one expert with weight 1, in the workspace
inline size_t shared_rows_bytes(int T) { return ((size_t)T * 4 + 255) / 256 * 256; }
inline size_t shared_routing_bytes(int T) { return 256 + 2 * shared_rows_bytes(T); }
void launch_identity_routing(int T, int32_t* offsets, int32_t* sorted_pair, float* w,
                             hipStream_t stream);
void launch_dequant(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                    const uint8_t* table_id, const TableArgs& ta, uint16_t* out, int blocks,
                    hipStream_t stream);

}  // namespace moeq
