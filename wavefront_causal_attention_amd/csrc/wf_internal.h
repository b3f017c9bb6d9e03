// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

constexpr int kMaxSlots = 64;      // context positions per round (bit per position)
constexpr int kMaxTablePages = 1024;  // T * pages_per_chunk, staged in LDS by attention
constexpr int kFp8Block = 64;      // tokens per fp8 scale block (restarts at each chunk)
constexpr int kMaxFp8Tiles = 4096;  // (context chunks) x (64-token blocks per chunk), fp8 attention
#ifndef WF_ATTN_BM
#define WF_ATTN_BM 256
#endif
constexpr int kAttnBM = WF_ATTN_BM;  // query rows per attention workgroup (32 per wave)
constexpr int kXcds = 8;           // MI355X: workgroup b runs on XCD b % 8

// Work-list entry of one attention workgroup: (slot, head, query tile) in the
// bit fields 31..26, 25..16 and 15..0 of a uint32 (slot < 64, head < 1024,
// query tile <= 0xFFFE), or kIdleWork for padding. All-ones cannot be a unit
// because the query-tile field of a real unit is at most 0xFFFE.
constexpr int32_t kIdleWork = -1;
__host__ __device__ inline int32_t pack_work(int s, int h, int q) {
    return (int32_t)(((uint32_t)s << 26) | ((uint32_t)h << 16) | (uint32_t)q);
}
__host__ __device__ inline int work_slot(int32_t w) { return (int)((uint32_t)w >> 26); }
__host__ __device__ inline int work_head(int32_t w) { return (int)(((uint32_t)w >> 16) & 1023u); }
__host__ __device__ inline int work_qtile(int32_t w) { return (int)((uint32_t)w & 0xFFFFu); }

// Page formats (per layer, physical page `phys`, head `h`, page token `t`,
// channel `d`). Both are made of 16-byte vectors of 8 bf16 values so that one
// 64-lane LDS-DMA instruction moves 1 KB of contiguous memory:
//   K: [phys][h][D/8][page_tokens][8]   element (t, d) at ((d/8)*pt + t)*8 + d%8
//   V: [phys][h][page_tokens/8][D][8]   element (t, d) at ((t/8)*D + d)*8 + t%8
// With fp8 Q/K the K pages hold e4m3 codes in 16-byte vectors of 16 channels:
//   K8: [phys][h][D/16][page_tokens][16]  byte (t, d) at ((d/16)*pt + t)*16 + d%16
// plus, per layer, the scale of each token's 64-token block
// kscale[phys][h][page_tokens] (fp32) and the chunk's K channel mean
// kmean[group][h][D] (fp32); the publish's scratch (sync words and fp64
// per-block K sums) follows them.
// Physical page of (context position p, page i of its chunk) = table[p*ppc + i].
__host__ __device__ inline int64_t k8_byte(int64_t page_head_base, int pt, int t, int d) {
    return page_head_base + ((int64_t)(d >> 4) * pt + t) * 16 + (d & 15);
}
__host__ __device__ inline int64_t k_elem(int64_t page_head_base, int pt, int t, int d) {
    return page_head_base + ((int64_t)(d >> 3) * pt + t) * 8 + (d & 7);
}
__host__ __device__ inline int64_t v_elem(int64_t page_head_base, int D, int t, int d) {
    return page_head_base + ((int64_t)(t >> 3) * D + d) * 8 + (t & 7);
}

// Fused RoPE + publish of `nslots` consecutive slots of one layer.
struct PublishArgs {
    const void* q;            // input rows, in_dtype; NULL: K/V only
    const void* k;
    const void* v;
    int64_t row_stride;       // elements between consecutive token rows
    void* q_out;              // [S+1][heads][N][D] bf16 or fp8
    float* q_scales;          // [S+1][heads][nblk] (fp8)
    void* kpage;              // this layer's K pages (format above)
    uint16_t* vpage;          // this layer's V pages (format above)
    float* kscale;            // fp8: per-token K scale [phys][head][pt]
    float* kmean;             // fp8: [group][head][D]
    double* kpart;            // fp8 scratch: [published slot][head][nblk][D] block sums of RoPE'd K
    const int32_t* table;     // page table [T][ppc]
    const double2* htab;      // RoPE row-axis (cos, sin) [frame_h][dh/2], fp64
    const double2* wtab;      // RoPE column-axis (cos, sin) [frame_w][dw/2], fp64
    const double* omega_t;    // RoPE time-axis frequencies [dt/2]
    int N, heads, D, pt, ppc, T, S;
    int frame_h, frame_w;
    int dt, dh, dw;
    int slot_first, nslots;
    int in_fp32;              // 1: input fp32, 0: bf16
    int nblk;                 // fp8 blocks per chunk
    int t0[kMaxSlots];        // RoPE time offset per published slot (ring == NULL)
    // live slots: the time offsets follow the pool's device round counter,
    // t0 = chunk_frames * (ring + t0_round - i) for published slot i, so a
    // captured launch stays right when it is replayed in later rounds
    const int64_t* ring;
    int64_t t0_round;         // first_round - slot_first
    int chunk_frames;
};
// RoPE time offset of published slot i of a launch
template <typename Args>
__device__ __forceinline__ int slot_t0(const Args& a, int i) {
    return a.ring ? a.chunk_frames * (int)(a.ring[0] + a.t0_round - i) : a.t0[i];
}

// Attention over the paged context for `nslots` query slots of one layer.
struct AttnArgs {
    const void* q;            // [S+1][heads][N][D]
    const float* q_scales;    // fp8: [S+1][heads][nblk]
    void* out;                // [S+1][N][heads*D]
    const void* kpage;        // this layer's K pages (format above)
    const uint16_t* vpage;    // this layer's V pages (format above)
    int32_t kbytes, vbytes;   // bytes of this layer's K / V regions (< 2^31)
    const float* kscale;      // fp8: per-token K scale [phys][head][pt]
    const float* kmean;       // fp8: [group][head][D]
    const int32_t* table;     // [T][ppc]
    const int32_t* work;      // per-workgroup (slot, head, qtile), -1 = idle
    int nwork;                // workgroups in the launch (multiple of kXcds)
    int N, heads, D, pt, ppc, T, S;
    int slot_first, nslots;
    int qtiles;               // query tiles per (slot, head)
    int out_fp32;
    int nblk;
    int all_live;             // 1: every slot reads the whole context (no mask)
    // occupied context positions: [0, anc) and [p2, T - s) (all-live: [p2,
    // end_all)); virtual position v maps to v < anc ? v : v + p2 - anc
    int anc, p2, end_all;
    float scale_log2;         // log2(e) / sqrt(D)
};

// QKV projection with RoPE + publish as its epilogue (bf16 pools), for
// `nslots` consecutive live slots of one layer.
constexpr int kProjTokens = 256;     // tokens per projection workgroup tile
constexpr int kProjChannels = 256;   // output channels per projection workgroup tile
constexpr int kProjMaxFrames = 8;    // latent frames one tile may touch (time table in LDS)
constexpr int kProjMaxRopeEntries = 2048;  // frame_h*dh/2 + frame_w*dw/2 (row/column tables in LDS)
struct ProjArgs {
    const void* x;            // hidden states [nslots * N][x_stride], bf16 or e4m3 codes
    int64_t x_stride;         // elements between token rows
    int32_t xbytes;           // bytes readable from x (< 2^31)
    const void* w;            // weight [3 * heads * D][hidden] ([out][in]), bf16 or e4m3 codes
    int32_t wbytes;           // bytes of w (< 2^31)
    const float* xs;          // e4m3 operands: scale per row of x [nslots * N]
    const float* ws;          // e4m3 operands: scale per output channel [3 * heads * D]
    const uint16_t* bias;     // [3 * heads * D] bf16, or NULL
    void* q_out;              // [S+1][heads][N][D] bf16
    void* kpage;              // this layer's K pages
    uint16_t* vpage;          // this layer's V pages
    const int32_t* table;     // page table [T][ppc]
    const float2* htab;       // RoPE row-axis (cos, sin) [frame_h][dh/2]
    const float2* wtab;       // RoPE column-axis (cos, sin) [frame_w][dw/2]
    const double* omega_t;    // RoPE time-axis frequencies [dt/2]
    int N, heads, D, pt, ppc, T, hidden;
    int frame_h, frame_w;
    int dt, dh, dw;
    int slot_first, nslots;
    int mtiles;               // token tiles per chunk
    int ctiles;               // 256-channel tiles of the 3 * heads * D outputs (the last may be half)
    int mrows;                // nslots * mtiles
    int g_ct, g_mt;           // XCD blocking: channel-tile groups x token-row groups = 8
    int t0[kMaxSlots];        // RoPE time offset per slot (ring == NULL)
    const int64_t* ring;      // as for PublishArgs
    int64_t t0_round;
    int chunk_frames;
};
int proj_frames_per_tile(int hw);
// f8: x and w are e4m3 codes with per-row scales (xs, ws), else bf16
hipError_t launch_project(const ProjArgs& a, bool f8, int nblocks, hipStream_t st);

constexpr int kQuantMaxCols = 8192;  // row width of the per-row e4m3 quantiser (held in registers)
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, int64_t x_stride, uint8_t* codes,
                             int64_t code_stride, float* scales, hipStream_t st);

// ring_dev == NULL: write the table for ring offset `ring`; else for the
// device counter's value + 1, then store that value back (one block)
hipError_t launch_page_table(int32_t* table, int T, int A, int ppc, int64_t ring, int64_t* ring_dev, int store_pos,
                             int store_anchor, hipStream_t st);
hipError_t launch_publish(const PublishArgs& a, bool fp8, hipStream_t st);
// wf_kv_publish_noalloc's scratch: one static device array per GPU
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_attention(const AttnArgs& a, bool fp8, hipStream_t st);
// blocks workgroups of 8 waves, each `steps` steps of 32 bf16 MFMAs per wave
hipError_t launch_mfma_calibrate(int32_t blocks, int32_t steps, float* out, hipStream_t st);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);

}  // namespace wf
