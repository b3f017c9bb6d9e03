// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

constexpr int kMaxSlots = 64;      // context positions per round (bit per position)
constexpr int kMaxTablePages = 1024;  // T * pages_per_chunk, staged in LDS by attention
constexpr int kFp8Block = 64;      // tokens per fp8 scale block (restarts at each chunk)

// Fused RoPE + publish of `nslots` consecutive slots of one layer.
struct PublishArgs {
    const void* q;            // input rows, in_dtype; NULL: K/V only
    const void* k;
    const void* v;
    int64_t row_stride;       // elements between consecutive token rows
    void* q_out;              // [S+1][heads][N][D] bf16 or fp8
    float* q_scales;          // [S+1][heads][nblk] (fp8)
    void* kpage;              // this layer's K pages: [phys][head][tok][D] (bf16 or fp8)
    uint16_t* vpage;          // this layer's V pages: [phys][head][D][tok] bf16
    float* kscale;            // fp8: [group][head][nblk]
    float* kmean;             // fp8: [group][head][D]
    const int32_t* table;     // page table [T][ppc]
    const float2* htab;       // RoPE row-axis (cos, sin) [frame_h][dh/2]
    const float2* wtab;       // RoPE column-axis (cos, sin) [frame_w][dw/2]
    const double* omega_t;    // RoPE time-axis frequencies [dt/2]
    int N, heads, D, pt, ppc, T, S;
    int frame_h, frame_w;
    int dt, dh, dw;
    int slot_first, nslots;
    int in_fp32;              // 1: input fp32, 0: bf16
    int nblk;                 // fp8 blocks per chunk
    int t0[kMaxSlots];        // RoPE time offset per published slot
};

// Attention over the paged context for `nslots` query slots of one layer.
struct AttnArgs {
    const void* q;            // [S+1][heads][N][D]
    const float* q_scales;    // fp8: [S+1][heads][nblk]
    void* out;                // [S+1][N][heads*D]
    const void* kpage;        // this layer's K pages
    const uint16_t* vpage;    // this layer's V pages (transposed per page)
    const float* kscale;      // fp8
    const float* kmean;       // fp8
    const int32_t* table;     // [T][ppc]
    int N, heads, D, pt, ppc, T, S;
    int slot_first, nslots;
    int qtiles;               // query tiles per (slot, head)
    int out_fp32;
    int nblk;
    float scale_log2;         // log2(e) / sqrt(D)
};

hipError_t launch_page_table(int32_t* table, int T, int A, int ppc, int64_t ring,
                             hipStream_t st);
hipError_t launch_publish(const PublishArgs& a, bool fp8, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, bool fp8, hipStream_t st);

}  // namespace wf
