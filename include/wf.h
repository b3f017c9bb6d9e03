/*
 * wf.h - C ABI of the wavefront-round attention library (libwf.so), gfx950.
 *
 * One wavefront round of chunk-wise causal attention in a Wan2.1-style DiT
 * layer (Wave Forcing, arXiv 2611.00859). In round k the S denoising slots
 * hold chunks k-s (s = 0 is the noisiest) and the store slot s = S holds the
 * chunk being written to clean history (hyper.ai summary, section "Method":
 * k = i + s; thelatestinai.com listing, Table 3: store = stage S). Every layer
 * attends over one ordered context (e-cogni.com.br article, "Como funciona"):
 *
 *     position:  0..A-1   | A..A+H-1               | A+H   | A+H+1 .. T-1
 *     contents:  anchor   | clean history, oldest  | store | slot S-1 .. slot 0
 *
 * with T = A+H+S+1. Attention is full inside a chunk and follows the mask
 * M_WF(s, j) = 1[j >= s] across live slots (hyper.ai, "Method"), so query slot
 * s reads exactly the context prefix [0, T-s) (anchor, history, store, and
 * slots S-1..s) and never a noisier slot.
 *
 * The library holds host state only (configuration, round index, readiness
 * bits) and allocates no device memory. The caller owns all of it: the pool
 * (K/V pages plus the RoPE tables, attention work lists, fp8 metadata and a
 * device round counter that wf_pool_create writes into it), the page table,
 * Q, O, scales and projection operands. Every launching call enqueues its
 * work on the given stream (a hipStream_t passed as void*, NULL for the
 * default stream) and returns without synchronising. A pool's launches must
 * run in the order they were issued (one stream, or streams ordered by
 * events), and calls on one handle must not overlap (a handle is not
 * thread-safe). No exception crosses the ABI; every call returns a status and
 * on any error launches nothing and changes no state.
 *
 * Slot numbering used by wf_kv_publish: slot s in [0, T) is context position
 * T-1-s. Slots 0..S are the live slots (s = S is the store); slots S+1..T-1
 * are the clean positions (history newest..oldest, then the anchor), which are
 * published directly only to seed a pool; in steady state they are filled by
 * wf_round_advance relabelling the store and history pages.
 */
#ifndef WF_H
#define WF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define WF_OK              0
#define WF_E_INVALID_ARG   1   /* bad pointer, index, dtype or range */
#define WF_E_SHAPE         2   /* configuration or buffer size not supported */
#define WF_E_NOT_READY     3   /* a required context position is not published */
#define WF_E_HIP           4   /* a HIP runtime call failed (see wf_last_error) */

/* live-slot visibility (wf_config.live_mask) */
#define WF_MASK_WAVEFRONT  0   /* M_WF(s, j) = 1[j >= s]: slot s reads the prefix [0, T-s)    */
#define WF_MASK_ALL_LIVE   1   /* every live slot reads every live slot: the whole context   */

/* element types */
#define WF_DTYPE_BF16      0
#define WF_DTYPE_FP32      1
#define WF_DTYPE_FP8_E4M3  2   /* OCP e4m3: max 448, no infinities */

typedef struct wf_config {
    int32_t S;               /* denoising slots, >= 1; the store is slot S          */
    int32_t anchor_chunks;   /* A >= 1: chunks of the initial anchor                */
    int32_t history_chunks;  /* H >= 0: bounded clean-history ring                  */
    int32_t heads;           /* attention heads per layer                           */
    int32_t head_dim;        /* d: 64 or 128                                        */
    int32_t num_layers;      /* layers sharing this pool and its page table        */
    int32_t chunk_frames;    /* latent frames per chunk                             */
    int32_t frame_h;         /* patch rows per latent frame                         */
    int32_t frame_w;         /* patch columns per latent frame                      */
    int32_t page_tokens;     /* tokens per page; divides the chunk, multiple of 8.
                                Limits: T = A+H+S+1 <= 64, T * pages per chunk
                                <= 1024, T * chunk tokens < 2^22 - 1              */
    int32_t in_dtype;        /* projected Q/K/V input: WF_DTYPE_BF16 | WF_DTYPE_FP32 */
    int32_t qk_dtype;        /* published Q/K: WF_DTYPE_BF16 | WF_DTYPE_FP8_E4M3
                                (fp8: T * ceil(chunk tokens / 64) <= 4096)         */
    int32_t rope_split[3];   /* (d_t, d_h, d_w), even, summing to head_dim          */
    int32_t first_round;     /* round index k of the pool's first round, >= 0; rounds
                                below S+H+A fill the pipeline (see live positions) */
    double  rope_theta;      /* RoPE base, e.g. 10000                               */
    int32_t live_mask;       /* WF_MASK_WAVEFRONT (default) | WF_MASK_ALL_LIVE: the
                                bidirectional live K/V of Rolling Forcing that the
                                pages contrast the wavefront mask with
                                (thelatestinai.com listing, Table 9); no tile is
                                skipped, for measuring what the mask saves         */
    int32_t total_chunks;    /* chunks in the video, 0 = unbounded stream; with C > 0
                                rounds run to C-1+S and the last S drain the pipeline */
} wf_config;

/*
 * Live positions. Chunk i enters slot 0 in round i and moves one stage per
 * round (k = i + s), is stored in round i+S and is clean afterwards: anchor
 * chunk a at anchor position a, later chunks in the history ring (the H most
 * recently stored). In the rounds that fill (k < S+H+A) and drain (k > C-1)
 * the pipeline some positions hold no chunk: they are not published, not
 * read and report chunk id -1 (thelatestinai.com listing, Figure 1 caption,
 * mentions the fill and its latency). A store that holds an anchor chunk is
 * published straight into that anchor's pages.
 */

typedef struct wf_handle wf_handle;

/*
 * Device memory a configuration needs. pool_bytes covers the K/V pages of all
 * layers, the fp8 scales and per-chunk K means (fp8 only) and the RoPE
 * tables; table_bytes is the int32 page table [T][pages_per_chunk].
 * Returns WF_E_SHAPE for an unsupported configuration.
 */
int wf_pool_bytes(const wf_config* cfg, size_t* pool_bytes, size_t* table_bytes);

/*
 * Bind a configuration to caller-allocated device memory (pool_dev of at least
 * pool_bytes, page_table_dev of at least table_bytes, both on the current
 * device). Writes the RoPE tables and the initial page table and waits for
 * them (blocking, setup only). Nothing is published yet. The library never
 * frees the caller's memory.
 */
int wf_pool_create(const wf_config* cfg, void* pool_dev, size_t pool_bytes,
                   int32_t* page_table_dev, size_t table_bytes, wf_handle** out);

/*
 * A handle with no device: it validates, schedules and tracks readiness
 * exactly like a device handle, but its launching calls enqueue nothing and
 * return WF_OK after every check and state change. For planning and for
 * testing the host state machine without a GPU; it never computes outputs.
 */
int wf_pool_create_host_model(const wf_config* cfg, wf_handle** out);

/* Frees host state only. */
void wf_pool_destroy(wf_handle* h);

/*
 * Fused 3D RoPE + K/V publish (hyper.ai summary, "Method": WaveRT publishes
 * K/V right after QKV projection and RoPE; paged delivery writes K/V straight
 * into ordered attention slots). One launch covers slots
 * [slot_first, slot_first + nslots) of one layer.
 *
 * q, k, v: device, in_dtype, row-major token rows; row (i*N + n) holds token n
 *          of slot slot_first + i, heads*head_dim contiguous elements starting
 *          at the pointer plus row * row_stride_elems. A fused [tokens, 3*h*d]
 *          projection output is q = base, k = base + h*d, v = base + 2*h*d with
 *          row_stride_elems = 3*h*d.
 * chunk_t0_host: optional host array [nslots] of RoPE time offsets (latent
 *          frame index of each slot's first frame); NULL takes
 *          chunk_frames * chunk id from the round schedule.
 * q_out:   device [S+1][heads][N][head_dim] bf16 (or fp8 e4m3 codes when
 *          qk_dtype is fp8, with q_scales device float [S+1][heads][ceil(N/64)]);
 *          rows of the published slots are written. q and q_out must both be
 *          NULL when the range includes clean slots (s > S), and may both be
 *          NULL to publish K/V only.
 * The K pages of the slot's context position receive RoPE'd K (bf16, or fp8
 * with per-64-token-block scales after subtracting the chunk's per-channel
 * mean); the V pages receive V in bf16. RoPE is computed in fp64 and every
 * published Q/K value is rounded once from it: bf16 to nearest even, fp8 as
 * the nearest-even e4m3 code of the fp64 quotient value / scale, scale =
 * fp32(block absmax) / 448, the mean the fp32 rounding of the fp64 mean.
 * Marks the slots published for this layer and round. WF_E_INVALID_ARG if a slot in the range holds no chunk in
 * this round (fill and drain rounds).
 */
int wf_kv_publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                  const void* q, const void* k, const void* v, int64_t row_stride_elems,
                  const int32_t* chunk_t0_host, void* q_out, float* q_scales, void* stream);

/*
 * wf_kv_publish for callers that cannot allocate device memory or must not
 * call hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it). Same arguments, checks and results as wf_kv_publish,
 * bit for bit; it allocates nothing. The scratch the fp8 publish needs (fp64
 * sums of RoPE'd K per 64-token block: nslots * heads * ceil(N/64) *
 * head_dim * 8 bytes) comes from one static device array of 16 MiB per GPU,
 * held until the process ends, instead of the pool's scratch region; larger
 * needs return WF_E_SHAPE and launch nothing (bf16 pools need none). Every
 * call on one GPU shares that GPU's array, so calls that may overlap on one
 * GPU (other streams, other threads, other pools) race: order them.
 */
int wf_kv_publish_noalloc(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                          const void* q, const void* k, const void* v, int64_t row_stride_elems,
                          const int32_t* chunk_t0_host, void* q_out, float* q_scales, void* stream);

/*
 * QKV projection with RoPE + publish as its epilogue (hyper.ai summary,
 * "Method": WaveRT publishes K/V right after the QKV projection and RoPE;
 * thelatestinai.com listing, Table 11: the projection maps the hidden state,
 * heads x 128 wide, to Q, K and V). One launch computes, for the live slots
 * [slot_first, slot_first + nslots) of one layer,
 *     qkv[n][o] = sum_c x[n][c] * w[o][c] + bias[o]
 * and publishes it as wf_kv_publish would publish that projection output
 * (RoPE on Q and K in fp32, bf16 pages and Q), without writing qkv to memory.
 *
 * x:      device bf16, row (i*N + n) = token n of slot slot_first + i, hidden
 *         contiguous elements at x + row * x_row_stride_elems (16-byte aligned
 *         rows).
 * hidden: input width, a multiple of 64.
 * w:      device bf16 [3*heads*head_dim][hidden], output channel o's weights
 *         contiguous (the [out][in] layout of a linear layer); outputs
 *         [0, h*d) are Q, [h*d, 2h*d) K, [2h*d, 3h*d) V, head-major.
 * bias:   device bf16 [3*heads*head_dim], 16-byte aligned, or NULL.
 * chunk_t0_host, q_out: as for wf_kv_publish (q_out required, bf16).
 * Only live slots (slot_first + nslots <= S+1). WF_E_SHAPE for fp8 pools,
 * heads*head_dim not a multiple of 128, a frame smaller than 1/32 of a
 * 256-token tile, or x or w of 2 GiB or more. Marks the slots published.
 */
int wf_qkv_project_publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                           const void* x, int64_t x_row_stride_elems, int32_t hidden, const void* w,
                           const void* bias, const int32_t* chunk_t0_host, void* q_out, void* stream);

/*
 * Per-row fp8 e4m3 quantisation of W8A8 operands (e-cogni.com.br, "Como
 * funciona": W8A8 quantisation of weights and activations; thelatestinai.com
 * listing, Table 6, the Sage+W8A8 backend). Row r of x (cols bf16 values at
 * x + r * x_row_stride_elems) gets the fp32 scale absmax / 448 (1 for an
 * all-zero row) and codes e4m3(x / scale), the quotient taken in IEEE fp32,
 * rounded to nearest even and saturated at +-448. Used on the hidden states
 * (one scale per token) and, once, on a weight [out][in] (one scale per
 * output channel). Inputs must be finite.
 *
 * x:      device bf16, 16-byte aligned, x_row_stride_elems a multiple of 8.
 * cols:   a multiple of 8, at most 8192.
 * codes:  device uint8 [rows][code_row_stride], 8-byte aligned,
 *         code_row_stride >= cols and a multiple of 8 (16 for a projection
 *         operand, whose rows must be 16-byte aligned).
 * scales: device float [rows].
 * rows = 0 launches nothing. Caller-owned memory; the work is enqueued on
 * stream. WF_E_INVALID_ARG for bad pointers or strides, WF_E_SHAPE for cols
 * out of range.
 */
int wf_quantize_rows_fp8(const void* x, int64_t rows, int32_t cols, int64_t x_row_stride_elems,
                         uint8_t* codes, int64_t code_row_stride, float* scales, void* stream);

/*
 * W8A8 form of wf_qkv_project_publish: the same launch and publish, with the
 * projection taken over e4m3 operands (v_mfma_f32_32x32x64_f8f6f4) and their
 * per-row scales,
 *     qkv[n][o] = x_scales[n] * w_scales[o] * sum_c x8[n][c] * w8[o][c] + bias[o]
 *
 * x8:       device e4m3 codes, row (i*N + n) = token n of slot slot_first + i,
 *           at x8 + row * x_row_stride (bytes, a multiple of 16), as written
 *           by wf_quantize_rows_fp8.
 * x_scales: device float [nslots*N], the scale of each x8 row, 16-byte aligned.
 * hidden:   a multiple of 128.
 * w8:       device e4m3 codes [3*heads*head_dim][hidden], 16-byte aligned.
 * w_scales: device float [3*heads*head_dim], 16-byte aligned.
 * bias, chunk_t0_host, q_out and the errors: as wf_qkv_project_publish.
 */
int wf_qkv_project_publish_w8a8(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                                const void* x8, int64_t x_row_stride, const float* x_scales, int32_t hidden,
                                const void* w8, const float* w_scales, const void* bias,
                                const int32_t* chunk_t0_host, void* q_out, void* stream);

/*
 * Wavefront attention over the paged context (hyper.ai summary, "Method":
 * M_WF(s, j) = 1[j >= s], full attention inside a chunk). One launch computes
 * O = softmax(Q K^T / sqrt(d)) V for query slots [slot_first, slot_first+nslots)
 * of one layer, each over its legal prefix; tiles of noisier slots are never
 * read. With live_mask = WF_MASK_ALL_LIVE every slot reads the whole context.
 *
 * q:        device, as q_out of wf_kv_publish (full [S+1] buffer).
 * q_scales: device fp8 query scales, NULL for bf16.
 * out:      device [S+1][N][heads*head_dim], out_dtype WF_DTYPE_BF16 or
 *           WF_DTYPE_FP32 (full-precision parity mode); rows of the computed
 *           slots are written.
 * Returns WF_E_NOT_READY, launching nothing, unless every context position the
 * slots read is published for this layer in this round (the readiness check
 * made just before attention); WF_E_INVALID_ARG if a requested slot holds no
 * chunk in this round. In fill and drain rounds each slot reads only the
 * positions that hold a chunk.
 */
int wf_attention_round(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                       const void* q, const float* q_scales, void* out, int32_t out_dtype,
                       void* stream);

/*
 * End the round: every chunk moves one position cleaner by rewriting the page
 * table, never by copying pages. The store's pages become the newest history,
 * the oldest history's pages are handed to slot 0 (re-published next round),
 * and the anchor stays. After r advances, non-anchor position p maps to page
 * group A + ((p - A + r) mod (H+S+1)); group g owns pages g*ppc .. g*ppc+ppc-1.
 * Requires the store published in every layer (WF_E_NOT_READY otherwise)
 * when the store holds a chunk; WF_E_INVALID_ARG past the last round of a
 * C-chunk video. Live slots become unpublished; history keeps its readiness; a
 * stored anchor chunk stays published at its anchor position.
 *
 * The rotation is driven by a round counter in the pool's device memory, from
 * which the publish launches of live slots also take their chunks' RoPE time
 * offsets (unless chunk_t0_host is given). A round's launches captured into a
 * HIP graph (publish or projection, attention, this advance) therefore stay
 * right when the graph is replayed in later rounds. Called on a stream that is
 * capturing, the advance is enqueued and the host state is left in the
 * captured round: call wf_round_replayed after every replay. Only steady
 * rounds (every position holds a chunk, the store holds no anchor chunk, this
 * round and the next) can be captured (WF_E_INVALID_ARG otherwise).
 */
int wf_round_advance(wf_handle* h, void* stream);

/*
 * Host bookkeeping for one replay of a captured round (see wf_round_advance):
 * the host state moves to the next round as the replayed advance left the
 * device, with the replayed round's store taken as published in every layer.
 * Launches nothing. WF_E_INVALID_ARG if no advance of this pool was captured,
 * for a round that is not steady, or for the last round of a video. Publish
 * and attention calls made while capturing update the host's readiness as if
 * they had run: replay the graph before relying on what they publish.
 */
int wf_round_replayed(wf_handle* h);

/*
 * Attention launch order (host only, no handle or device needed): the list
 * the pool uploads for query slots [slot_first, slot_first + nslots), i.e.
 * what workgroup b of an attention launch computes. Entry b is
 * (slot << 26) | (head << 16) | query_tile, or -1 for an idle workgroup;
 * workgroup b runs on XCD b % 8. The (slot, head, query tile) units are cut
 * into 8 pieces of equal key-chunk cost, one per XCD, and each piece is packed
 * onto cus_per_xcd CUs and listed by planned start time. *count receives the
 * length (a multiple of 8); units (capacity entries) may be NULL to query it.
 */
int wf_attention_work_list(const wf_config* cfg, int32_t slot_first, int32_t nslots, int32_t cus_per_xcd,
                           int32_t* units, int64_t capacity, int64_t* count);

/* Host queries (no device access). */
int wf_round_index(const wf_handle* h, int64_t* k);
int wf_schedule_chunk_ids(const wf_handle* h, int64_t* ids /* [T], -1 = no chunk */);
int wf_page_table_host(const wf_handle* h, int32_t* table /* [T * pages_per_chunk] */);
int wf_ready_mask(const wf_handle* h, int32_t layer, uint64_t* mask /* bit p = position p */);
/* Pool geometry, out[12]: N, T, pages_per_chunk, K region offset, V region
 * offset, K bytes per layer, V bytes per layer, fp8 K-scale region offset,
 * K-scale bytes per layer, fp8 K-mean region offset, K-mean bytes per layer,
 * 64-token blocks per chunk. Byte offsets are into the pool. */
int wf_geometry(const wf_handle* h, int64_t* out);
/*
 * Matrix-core calibration for the attention roofline: `blocks` workgroups of
 * 8 waves (one per CU, as the attention kernel runs), each wave issuing
 * `steps` x 32 v_mfma_f32_32x32x16_bf16 on nonzero register operands, the
 * attention step's MFMA mix (16 into two score blocks, 16 into four output
 * blocks). FLOPs = blocks * 8 * steps * 32 * 32768. Timed by the caller on
 * `stream`, it gives the dense bf16 rate this GPU sustains at the clock it
 * holds under MFMA load, the attention kernel's attainable ceiling (no memory
 * traffic, no softmax). out: device float [blocks * 512], a checksum per lane.
 */
int wf_mfma_calibrate(int32_t blocks, int32_t steps, float* out, void* stream);

/*
 * HBM calibration for the publish roofline: copies `bytes` (a positive
 * multiple of 16) from device buffer src to device buffer dst (both 16-byte
 * aligned, not overlapping) with a streaming kernel that does nothing else:
 * two 16-byte non-temporal loads and plain stores per thread. Timed by the
 * caller on `stream`, (2 * bytes) / time is the read+write rate this GPU
 * reaches for that byte count, the attainable ceiling of an HBM-bound kernel
 * with the same mix. WF_E_INVALID_ARG (nothing launched) for a null pointer,
 * a size that is not a positive multiple of 16 or a misaligned pointer.
 */
int wf_stream_copy_calibrate(const void* src, void* dst, int64_t bytes, void* stream);

const char* wf_status_string(int status);
const char* wf_last_error(const wf_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* WF_H */
