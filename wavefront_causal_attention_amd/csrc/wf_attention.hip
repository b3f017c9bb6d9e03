// Wavefront attention over the paged K/V context, gfx950: bf16 MFMA, or fp8
// e4m3 MFMA for QK^T with bf16 PV.
//
// One launch covers every (query slot, head, query tile) of the round. Query
// slot s reads the context prefix [0, (T-s)*N) - anchor, clean history, store
// and the live slots that are not noisier than s - which is exactly the mask
// M_WF(s, j) = 1[j >= s] with full attention inside each chunk (Wave Forcing,
// hyper.ai summary, section "Method"; e-cogni.com.br, "Como funciona"). The
// key loop simply stops at the prefix end, so masked slot pairs are skipped as
// whole tiles and their pages are never read. With the all-live mask (the
// bidirectional live K/V the pages contrast it with) every slot reads the
// whole context.
//
// Per workgroup: 256 query rows of one (slot, head), 8 waves of 32 rows, one
// workgroup per CU. Per 64-key tile, each wave computes
//   S^T[key][query] = K Q^T      (v_mfma_f32_32x32x16_bf16, K from LDS, Q in VGPRs)
//   O^T[d][query]  += V^T P^T    (V^T from LDS, P^T from the S^T accumulators)
// so a lane owns one query row throughout: the softmax max and sum are in-lane
// except one exchange between the two 32-lane halves (v_permlane32_swap). The
// K row that feeds accumulator row r is key r with bits 2 and 3 swapped, which
// leaves each lane the scores of exactly the keys its half supplies to the PV
// MFMA's B operand, so P^T is packed in place with no cross-lane moves.
//
// Tiles arrive by LDS DMA (buffer_load ... lds): each instruction moves 1 KB
// of contiguous page memory, keys past the legal prefix read out of range and
// land as zeros. Every K/V tile brought into LDS feeds all 8 waves (256 query
// rows), which halves the L2-to-LDS traffic per flop of a 128-row tile. K and
// V each cycle through NSTG tile buffers: a tile's DMA is issued NSTG-1 steps
// before it is read, and a step waits only for the previous step's DMA. K runs
// one tile ahead of V so that S(t+1) = K(t+1) Q^T is issued while the softmax
// of tile t runs, and PV(t) while the row max of tile t+1 runs.
//
// On gfx950 the VALU work of the softmax (exp2, max, bf16 packing, row sums)
// does not overlap MFMAs on the same SIMD, also across waves, so the step is
// kept to one MFMA per LDS fragment read and the fewest VALU instructions per
// score (one FMA + one exp2, a half v_max3, a half v_cvt_pk, a half v_dot2).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = kAttnBM;     // query rows per workgroup
constexpr int NW = BM / 32;     // waves per workgroup
constexpr int NTH = 64 * NW;    // threads per workgroup
constexpr int BN = 64;          // keys per tile
#ifndef WF_ATTN_STAGES
#define WF_ATTN_STAGES 3
#endif
constexpr int NSTG = WF_ATTN_STAGES;   // K and V tile buffers each
// A step waits only for the DMA issued one step earlier, so the tiles a step
// reads were issued at least two steps before it: three stages at least.
static_assert(NSTG >= 3 && NSTG <= 4, "3 or 4 tile stages");
static_assert(NW >= 4 && NW <= 8 && BM % 32 == 0, "4 to 8 waves of 32 query rows");
constexpr int kRescaleLog2 = 8; // running max may lag the true max by up to 2^8
// Buffer offset past every region (each is under 2^31 bytes): loads zeros.
// The in-tile addends of a DMA are below 2^31 as well, so kOOB plus any of
// them stays out of range without wrapping.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Wait until at most n (wave-uniform, 0..7) vector memory operations of this
// wave are outstanding: the n issued last may still be in flight.
__device__ __forceinline__ void wait_vmem_upto(int n) {
    switch (n) {
        case 1: wait_vmem_n<1>(); break;
        case 2: wait_vmem_n<2>(); break;
        case 3: wait_vmem_n<3>(); break;
        case 4: wait_vmem_n<4>(); break;
        case 5: wait_vmem_n<5>(); break;
        case 6: wait_vmem_n<6>(); break;
        case 7: wait_vmem_n<7>(); break;
        default: wait_vmem(); break;
    }
}

// Workgroup barrier for the tile pipeline. __syncthreads() adds a release
// fence, which waits for every outstanding LDS DMA (vmcnt(0)) and would drain
// the prefetches in flight; here each wave has already waited for the DMA the
// next step reads, and its own LDS reads have returned (lgkmcnt(0)), so a bare
// s_barrier orders the buffers. The memory clobber keeps the compiler from
// moving LDS or buffer accesses across it.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Tile buffers: separate LDS arrays, addressed with compile-time indices in
// the steady-state loop, so the compiler can tell the buffer a DMA fills from
// the ones being read and does not wait for the DMA before reading. Sized for
// the largest head dimension (a K or V tile of 64 keys x 128 bf16 channels).
constexpr int kTileElems = BN * 128;
__shared__ __align__(16) uint16_t g_kt0[kTileElems];
__shared__ __align__(16) uint16_t g_kt1[kTileElems];
__shared__ __align__(16) uint16_t g_kt2[kTileElems];
__shared__ __align__(16) uint16_t g_kt3[kTileElems];
__shared__ __align__(16) uint16_t g_vt0[kTileElems];
__shared__ __align__(16) uint16_t g_vt1[kTileElems];
__shared__ __align__(16) uint16_t g_vt2[kTileElems];
__shared__ __align__(16) uint16_t g_vt3[kTileElems];
__shared__ int g_ptab[kMaxTablePages];
// element offset of (page, head) for each virtual page of the slot's context
__shared__ uint32_t g_pbase[kMaxTablePages];
__shared__ float g_stab[kMaxFp8Tiles];   // fp8: key scale of every tile of the prefix

template <int I>
__device__ __forceinline__ uint16_t* kbuf() {
    if constexpr (I == 0) return g_kt0;
    else if constexpr (I == 1) return g_kt1;
    else if constexpr (I == 2) return g_kt2;
    else return g_kt3;
}
template <int I>
__device__ __forceinline__ uint16_t* vbuf() {
    if constexpr (I == 0) return g_vt0;
    else if constexpr (I == 1) return g_vt1;
    else if constexpr (I == 2) return g_vt2;
    else return g_vt3;
}
__device__ __forceinline__ uint16_t* kbuf_rt(int i) {
    return i == 0 ? kbuf<0>() : i == 1 ? kbuf<1>() : i == 2 ? kbuf<(NSTG > 2 ? 2 : 0)>() : kbuf<(NSTG > 3 ? 3 : 0)>();
}
__device__ __forceinline__ uint16_t* vbuf_rt(int i) {
    return i == 0 ? vbuf<0>() : i == 1 ? vbuf<1>() : i == 2 ? vbuf<(NSTG > 2 ? 2 : 0)>() : vbuf<(NSTG > 3 ? 3 : 0)>();
}

#ifndef WF_SCHED
#define WF_SCHED 1
#endif
#ifndef WF_SCHED_PRE
#define WF_SCHED_PRE 4
#endif
#ifndef WF_SCHED_VS
#define WF_SCHED_VS 5
#endif
#ifndef WF_SCHED_VP
#define WF_SCHED_VP 2
#endif
// Scheduling template for one pipeline step: LDS reads issued ahead, each
// MFMA of S(t+1) then of PV(t) followed by the next LDS read and a few VALU
// instructions of the softmax (WF_SCHED=0 leaves the order to the compiler;
// the counts are tuning knobs, measured flat within a few percent).
template <int D, bool FP8>
__device__ __forceinline__ void sched_pipeline() {
#if WF_SCHED == 1
    constexpr int NS = FP8 ? 2 * (D / 64) : 2 * (D / 16);
    constexpr int NP = 4 * (D / 32);
    __builtin_amdgcn_sched_group_barrier(0x100, WF_SCHED_PRE, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, WF_SCHED_VS, 0);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, WF_SCHED_VP, 0);
    }
#endif
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ i32x8 as_i32x8(uint4 a, uint4 b) {
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Unsigned division by a run-time invariant divisor d >= 1 for any 32-bit
// numerator: multiply by a precomputed 32-bit factor and shift (Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", 1994,
// section 4). Branch-free, so page lookups can be scheduled among MFMAs.
struct FastDiv {
    uint32_t m;
    uint32_t s1, s2;
};
__device__ __forceinline__ FastDiv make_fastdiv(uint32_t d) {
    const uint32_t l = d > 1 ? 32 - __clz(d - 1) : 0;              // ceil(log2 d)
    const uint64_t m = ((uint64_t)1 << 32) * (((uint64_t)1 << l) - d) / d + 1;
    return FastDiv{(uint32_t)m, l < 1 ? l : 1u, l > 1 ? l - 1 : 0u};
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    const uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// FP8: Q and K are e4m3 codes with per-64-token-block scales and the chunk's
// K mean removed; QK^T runs on v_mfma_f32_32x32x64_f8f6f4 and each raw score
// becomes s_k * (q8 . k8) + q8 . mean(chunk); the query scale is folded into
// the softmax's exp2 constant. V and PV stay bf16. Key tiles are the 64-token
// quantisation blocks of each chunk, so a tile has one key scale and one
// chunk mean: the affine dequantisation folds into the exp2 argument (one FMA
// per score, as for bf16) and the row max is taken on the raw accumulator
// (the scale is positive). The last block of a chunk is partial unless 64
// divides the chunk; its missing keys are masked.

// Scores of one key tile: the S^T accumulators and, for fp8, the tile's key
// scale and this lane's chunk bias.
struct TileS {
    f32x16 s[2];
    float sk, b;
};
template <int D, bool FP8>
__global__ __launch_bounds__(NTH, NW == 4 ? 2 : 1) void attn_kernel(AttnArgs a) {
    constexpr int DC = D / 8;       // 16-byte channel vectors per key
    constexpr int KSTEPS = D / 16;  // MFMA k-steps of QK^T
    constexpr int DB = D / 32;      // 32-wide d blocks of the output
    constexpr int VDH = D / 64;     // 64-channel halves of a V key-chunk
    // DMA instructions per tile: K is [channel vector][key][16 B] with one
    // instruction per vector (D/8 bf16 or D/16 fp8 vectors), V is [key chunk
    // of 8][d][8] with one instruction per 64 channels of a chunk (8 * VDH).
    constexpr int KV = FP8 ? D / 16 : DC;
    constexpr int KPW = (KV + NW - 1) / NW;          // K instructions per wave (upper bound)
    constexpr int VCW = 8 / NW;                      // V key chunks per wave
    static_assert(KV <= NW * KPW && 8 % NW == 0 && D * BN <= kTileElems, "tile split");
    int* const ptab = g_ptab;

    const int tid = threadIdx.x;
    const int32_t unit = a.work[blockIdx.x];
    if (unit == kIdleWork) return;                 // padding of the per-XCD work lists
    const int s = work_slot(unit);
    const int head = work_head(unit);
    const int qt = work_qtile(unit);
    const int N = a.N, pt = a.pt, ppc = a.ppc;
    // context chunks slot s reads: the occupied positions [0, anc) and [p2,
    // end) (every position of the prefix in steady rounds), visited through a
    // virtual position v -> v < anc ? v : v + gap
    const int gap = a.p2 - a.anc;
    const int nctx = a.anc + (a.all_live ? a.end_all : a.T - s) - a.p2;
    const int nkeys = nctx * N;                    // legal keys of slot s
    // bf16: tiles cover the flat prefix; fp8: tpc tiles per chunk
    const int tpc = FP8 ? (N + BN - 1) / BN : 1;
    const int ntiles = FP8 ? nctx * tpc : (nkeys + BN - 1) / BN;
    const FastDiv tdiv = make_fastdiv((uint32_t)tpc);

    for (int i = tid; i < a.T * ppc; i += NTH) ptab[i] = a.table[i];
    // Page base of every virtual page: the context's occupied positions
    // renumbered without the gap, each page's (page, head) block in elements
    // (the same for K and V; K bytes = KB x elements, V bytes = 2 x elements).
    // Below 2^30 because every page region is under 2 GiB.
    for (int i = tid; i < nctx * ppc; i += NTH) {
        const int pp = i < a.anc * ppc ? i : i + gap * ppc;
        g_pbase[i] = (uint32_t)(((int64_t)a.table[pp] * a.heads + head) * pt * D);
    }

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int qrow = qt * BM + wave * 32 + l32;
    // A wave whose 32 query rows all lie past the chunk (in the last query
    // tile of a chunk that is not a multiple of BM rows) runs the pipeline
    // without its MFMA and softmax work: it issues its share of every tile's
    // DMA and takes every wait and barrier, so the workgroup's schedule is
    // unchanged, and its SIMD runs the other wave alone.
    const bool idle = qt * BM + wave * 32 >= N;
    // K row read for accumulator row l32: bits 2 and 3 swapped. Element j of a
    // lane's S^T accumulator block kb then holds key 32*kb + key_in_block(j) +
    // 8*hf, with key_in_block(j) = 16*(j/8) + j%8.
    const int krow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.kpage), (short)0, a.kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.vpage), (short)0, a.vbytes, 0x00020000);
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    const float c = a.scale_log2;
    float cl = c;                                  // exp2 constant of this lane's row

    // Q^T operand fragments: lane holds Q[qrow][16*ks + 8*hf .. +7] (bf16) or
    // the 32 codes Q8[qrow][64*ks + 32*hf .. +31] (fp8)
    bf16x8 qf[FP8 ? 1 : KSTEPS];
    i32x8 qf8[FP8 ? D / 64 : 1];
    if constexpr (!FP8) {
        const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                             (((int64_t)s * a.heads + head) * N + min(qrow, N - 1)) * D + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 u = *reinterpret_cast<const uint4*>(qb + 16 * ks);
            if (qrow >= N) u = make_uint4(0, 0, 0, 0);
            qf[ks] = as_bf16x8(u);
        }
    } else {
        const uint8_t* qb = static_cast<const uint8_t*>(a.q) +
                            (((int64_t)s * a.heads + head) * N + min(qrow, N - 1)) * D + 32 * hf;
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
            uint4 u0 = *reinterpret_cast<const uint4*>(qb + 64 * ks);
            uint4 u1 = *reinterpret_cast<const uint4*>(qb + 64 * ks + 16);
            if (qrow >= N) u0 = u1 = make_uint4(0, 0, 0, 0);
            qf8[ks] = as_i32x8(u0, u1);
        }
        const float sq = a.q_scales[((int64_t)s * a.heads + head) * a.nblk + min(qrow, N - 1) / kFp8Block];
        cl = c * sq;
    }

    // Tiles of the next K and V DMA. This lane loads key row `lane` of each K
    // tile, this wave key chunks wave*VCW .. of each V tile. A chunk is ppc
    // whole pages of pt tokens, so flat key g is token g % pt of context page
    // g / pt.
    int ktile = 0, vtile = 0;
    // flat virtual key index of offset o (< 64) in tile t, and whether it is legal
    auto tile_key = [&](int t, int o, bool& ok) -> int {
        if constexpr (FP8) {
            const int c = (int)fast_div((uint32_t)t, tdiv);
            const int o64 = (t - c * tpc) * BN + o;
            ok = c < nctx && o64 < N;
            return c * N + o64;
        } else {
            const int g = t * BN + o;
            ok = g < nkeys;
            return g;
        }
    };
    // Virtual page and token of a legal flat key g (< 2^22, checked on the
    // host): floor((g + 1/2) / pt) in fp32 is exact there, since the relative
    // error of the two roundings stays below the 1/(2 pt) margin to the next
    // integer; this keeps the 32-bit multiplies off the per-tile VALU budget.
    const float rpt = 1.0f / (float)pt;
    const float rpt_half = 0.5f * rpt;
    auto page_tok = [&](uint32_t g, uint32_t& tok) -> uint32_t {
        const uint32_t pidx = (uint32_t)__builtin_fmaf((float)g, rpt, rpt_half);
        tok = g - __umul24(pidx, (uint32_t)pt);
        return pidx;
    };

    // K instructions of this wave: vectors wave*KPW .. (wave+1)*KPW-1 below KV
    const int kmine = max(0, min(KPW, KV - wave * KPW));
    // vector memory instructions one full step issues in this wave (the same
    // in every wave when KV % NW == 0)
    const int ndma = kmine + VCW * VDH;
    constexpr int kDmaUniform = KV % NW == 0 ? KPW + VCW * VDH : -1;
    auto wait_older_dma = [&]() {
        if constexpr (kDmaUniform < 0) wait_vmem_upto(ndma);
        else wait_vmem_n<kDmaUniform>();
    };

    __syncthreads();                               // ptab visible
    if constexpr (FP8) {
        // key scale of every tile: the scale of its block's first token
        for (int i = tid; i < ntiles; i += NTH) {
            const int c = (int)fast_div((uint32_t)i, tdiv);
            const int n = (i - c * tpc) * BN;
            const int pg = n / pt, tok = n - pg * pt;
            const int pos = c < a.anc ? c : c + gap;
            g_stab[i] = a.kscale[((int64_t)ptab[pos * ppc + pg] * a.heads + head) * pt + tok];
        }
    }
    // Offsets of the next tile's DMA are computed one tile ahead (page-table
    // lookup in LDS plus the page arithmetic), right after the previous DMA is
    // issued, so that their latency overlaps the step's MFMA work and the DMA
    // issue after the barrier is a handful of scalar and buffer instructions.
    uint32_t koff = kOOB;                          // this lane's key row of the next K tile
    uint32_t voff[VCW];                            // this wave's key chunks of the next V tile
    auto k_addr = [&]() {
        bool ok;
        const int g = tile_key(ktile, lane, ok);
        uint32_t tok;
        const uint32_t pidx = page_tok(ok ? (uint32_t)g : 0u, tok);   // the lookup stays in the table
        const uint32_t off = g_pbase[pidx] * (FP8 ? 1u : 2u) + tok * 16u;
        koff = ok ? off : kOOB;
    };
    // a V key chunk is wave-uniform: its page split runs on the scalar unit
    const FastDiv pdiv = make_fastdiv((uint32_t)pt);
    auto v_addr = [&](int i) {
        bool ok;
        const int g = tile_key(vtile, 8 * (wave * VCW + i), ok);
        const uint32_t gi = ok ? (uint32_t)g : 0u;
        const uint32_t pidx = fast_div(gi, pdiv);
        const uint32_t tok = gi - pidx * (uint32_t)pt;
        const uint32_t base = __builtin_amdgcn_readfirstlane(g_pbase[pidx]);
        const uint32_t off = base * 2u + tok * (uint32_t)(2 * D);
        voff[i] = ok ? off : kOOB;
    };
    k_addr();
#pragma unroll
    for (int i = 0; i < VCW; ++i) v_addr(i);

    auto dma_k = [&](uint16_t* kl) {
        // one instruction per 16-byte vector: bf16 K [vector][key][8 ch],
        // fp8 K8 [vector][key][16 ch]
        uint8_t* kb8 = reinterpret_cast<uint8_t*>(kl);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int vec = wave * KPW + i;
            if (KV % NW == 0 || i < kmine)
                dma16(krs, kb8 + vec * BN * 16, koff + (uint32_t)(vec * pt * 16));
        }
        ++ktile;
        k_addr();
    };
    auto dma_v = [&](uint16_t* vl) {
#pragma unroll
        for (int i = 0; i < VCW; ++i) {
            const int kc = wave * VCW + i;
#pragma unroll
            for (int h = 0; h < VDH; ++h)
                dma16(vrs, vl + (kc * D + 64 * h) * 8, voff[i] + (uint32_t)((64 * h + lane) * 16));
        }
        ++vtile;
#pragma unroll
        for (int i = 0; i < VCW; ++i) v_addr(i);
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    float m_run = -INFINITY;   // running max of raw scores (may lag by < 2^8 in exp2 units)
    float l_run = 0.f;         // this lane's partial row sum (of the bf16-rounded weights)

    auto compute_s = [&](const uint16_t* kl, TileS& T) {
        f32x16 (&S)[2] = T.s;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) S[kb][j] = 0.f;
        if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 ka = as_bf16x8(
                        *reinterpret_cast<const uint4*>(kl + ((2 * ks + hf) * BN + 32 * kb + krow) * 8));
                    S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], S[kb], 0, 0, 0);
                }
        } else {
            const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kl);
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint4 u0 = *reinterpret_cast<const uint4*>(kb8 + ((4 * ks + 2 * hf) * BN + 32 * kb + krow) * 16);
                    const uint4 u1 = *reinterpret_cast<const uint4*>(kb8 + ((4 * ks + 2 * hf + 1) * BN + 32 * kb + krow) * 16);
                    S[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_i32x8(u0, u1), qf8[ks], S[kb],
                                                                            0, 0, 0, 0, 0, 0);
                }
        }
    };
    // fp8: this lane's bias q8 . mean(chunk) for the chunk of the tile
    // dequantised next; recomputed only when tiles enter a new chunk.
    int bchunk = 0;
    float bcur = 0.f;
    auto chunk_bias = [&](int vpos) -> float {
        if (vpos >= nctx) return 0.f;
        const int pos = vpos < a.anc ? vpos : vpos + gap;
        const int g = ptab[pos * ppc] / ppc;
        const float* mu = a.kmean + ((int64_t)g * a.heads + head) * D + 32 * hf;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll 1
            for (int w = 0; w < 8; ++w) {
                const float4 m4 = *reinterpret_cast<const float4*>(mu + 64 * ks + 4 * w);
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(qf8[ks][w], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(qf8[ks][w], true);
                acc = fmaf(lo[0], m4.x, acc);
                acc = fmaf(lo[1], m4.y, acc);
                acc = fmaf(hi[0], m4.z, acc);
                acc = fmaf(hi[1], m4.w, acc);
            }
        const uint32_t ab = __float_as_uint(acc);
        const auto sw = __builtin_amdgcn_permlane32_swap(ab, ab, false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    // Advanced at the end of a step, outside the MFMA/VALU interleaving,
    // since it branches and loads the means only when tiles enter a new chunk.
    auto chunk_advance = [&](int tile) {
        if constexpr (FP8) {
            const int c = (int)fast_div((uint32_t)tile, tdiv);
            if (c != bchunk) {
                bchunk = c;
                bcur = chunk_bias(c);
            }
        }
    };
    // Row max of tile `tile`, then the running-max update; O and l are
    // rescaled only when the max grows by more than 2^8 in exp2 units (a
    // wave-uniform, rare branch). bf16: only the last tile of a prefix can
    // hold keys past it; the masking variant (maskc = true) is instantiated
    // outside the main loop only, so the steady-state loop carries no masking
    // code. fp8: the last tile of every chunk is masked when partial (a
    // uniform branch), and the max of the raw accumulator maps through the
    // tile's affine dequantisation.
    auto update_max = [&](TileS& T, int tile, auto maskc) {
        f32x16 (&S)[2] = T.s;
        constexpr bool kMaskBf16 = !FP8 && decltype(maskc)::value;
        int rem = BN;                                  // legal keys of this tile (wave-uniform)
        if constexpr (FP8) rem = N - (tile - (int)fast_div((uint32_t)tile, tdiv) * tpc) * BN;
        else if constexpr (kMaskBf16) rem = nkeys - tile * BN;
        if (FP8 || kMaskBf16) {
            if (rem < BN) {
                const int lim = rem - 8 * hf;          // keys >= lim (lane-relative) are masked
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = 32 * kb + 16 * (j >> 3) + (j & 7);
                        S[kb][j] = key < lim ? S[kb][j] : -INFINITY;
                    }
            }
        }
        float mx = S[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, S[kb][j]);
        const uint32_t mb = __float_as_uint(mx);
        const auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        if constexpr (FP8) {
            T.sk = g_stab[tile];
            T.b = bcur;
            mx = fmaf(mx, T.sk, T.b);
        }
        const float m_new = fmaxf(m_run, mx);
        if (__any((m_new - m_run) * cl > (float)kRescaleLog2)) {
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * cl);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
    };
    // P = exp2(S*c - m*c) rounded to bf16; the row sum adds the same rounded
    // values (v_dot2 with (1, 1)) so the weights applied to V are normalised
    // exactly. With the permuted K rows, elements 8g..8g+7 of accumulator
    // block kb are keys 16*(2*kb+g) + 8*hf + 0..7: the B operand of PV group
    // G = 2*kb+g as it stands, matching V^T in LDS (key chunk 2*G + hf).
    auto exp_pack = [&](TileS& T, bf16x8 (&P)[4]) {
        f32x16 (&S)[2] = T.s;
        // exp2 argument = A * acc + B: bf16 A = c, B = -m c; fp8 A = s_k c,
        // B = (bias - m) c (the tile's affine dequantisation folded in)
        const float A = FP8 ? T.sk * cl : cl;
        const float B = FP8 ? (T.b - m_run) * cl : -m_run * cl;
        uint32_t w[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[kb][j], A, B));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[kb][j + 1], A, B));
                w[kb][j >> 1] = pack_bf16x2(p0, p1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[kb][j >> 1]),
                                                        kOnes, l_run, false);
            }
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const uint32_t* src = w[G >> 1] + 4 * (G & 1);
            P[G] = as_bf16x8(make_uint4(src[0], src[1], src[2], src[3]));
        }
    };
    auto compute_pv = [&](const uint16_t* vl, const bf16x8 (&P)[4]) {
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 va = as_bf16x8(
                    *reinterpret_cast<const uint4*>(vl + ((2 * G + hf) * D + 32 * db + l32) * 8));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[G], oacc[db], 0, 0, 0);
            }
    };
    // One pipeline step for tile t: K(t+NSTG) and V(t+NSTG-1) are fetched
    // into the buffers that K(t) and V(t-1) left free last step, while S(t+1)
    // is computed next to the softmax of tile t, then PV(t) runs next to the
    // max of tile t+1. Tile j lives in K and V buffer j % NSTG. At the end the
    // wave waits only for the DMA issued one step earlier (K(t+2) and V(t+1),
    // needed next step) and leaves this step's in flight. S(t+1) is computed
    // even past the last tile (from stale LDS, never used) so that its MFMAs
    // share a basic block with the softmax.
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    using Main = std::integral_constant<bool, true>;   // every fetch is issued; tile t+1 is not the last
    using Tail = std::integral_constant<bool, false>;  // one of the last steps
    auto step = [&](int t, const uint16_t* k_next, uint16_t* k_fill, const uint16_t* v_cur,
                    uint16_t* v_fill, TileS& Scur, TileS& Snext,
                    auto mainc, auto idlec) __attribute__((always_inline)) {
        constexpr bool kMain = decltype(mainc)::value;
        tile_barrier();
        if (kMain || t + NSTG < ntiles) dma_k(k_fill);
        if (kMain || t + NSTG - 1 < ntiles) dma_v(v_fill);
        if constexpr (decltype(idlec)::value) {
            if constexpr (kMain) wait_older_dma();
            else wait_vmem();
            return;
        }
        bf16x8 P[4];
        compute_s(k_next, Snext);
        exp_pack(Scur, P);
        compute_pv(v_cur, P);
        if constexpr (kMain) {
            update_max(Snext, t + 1, NoMask{});
            sched_pipeline<D, FP8>();
            wait_older_dma();
        } else {
            sched_pipeline<D, FP8>();
            if (t + 1 < ntiles) update_max(Snext, t + 1, Mask{});
            wait_vmem();
        }
        chunk_advance(t + 2);
    };

    // the pipeline, instantiated for computing and for idle waves: the same
    // DMA, waits and barriers in the same order in both
    auto run = [&](auto idlec) __attribute__((always_inline)) {
        // prologue: K(0..NSTG-1) and V(0..NSTG-2) in flight, then S(0)
        static_for<0, NSTG>([&](auto j) __attribute__((always_inline)) {
            if (j < ntiles) dma_k(kbuf<j>());
            if (j + 1 < NSTG && j < ntiles) dma_v(vbuf<j>());
        });
        wait_vmem();
        __syncthreads();
        TileS SA, SB;
        if constexpr (FP8) bcur = chunk_bias(0);
        if constexpr (!decltype(idlec)::value) {
            compute_s(kbuf<0>(), SA);
            update_max(SA, 0, Mask{});
            chunk_advance(1);
        }
        int t = 0;
        // steady state, NSTG steps per iteration with fixed buffers: step t + j
        // reads K buffer (j+1) % NSTG and V buffer j, fills K buffer j and V
        // buffer (j-1) % NSTG; the score accumulators alternate SA/SB
        if constexpr (NSTG % 2 == 0) {
            for (; t + 2 * NSTG - 1 < ntiles; t += NSTG)
                static_for<0, NSTG>([&](auto j) __attribute__((always_inline)) {
                    constexpr int J = decltype(j)::value;
                    if constexpr (J % 2 == 0)
                        step(t + J, kbuf<(J + 1) % NSTG>(), kbuf<J>(), vbuf<J>(), vbuf<(J + NSTG - 1) % NSTG>(),
                             SA, SB, Main{}, idlec);
                    else
                        step(t + J, kbuf<(J + 1) % NSTG>(), kbuf<J>(), vbuf<J>(), vbuf<(J + NSTG - 1) % NSTG>(),
                             SB, SA, Main{}, idlec);
                });
        } else {
            // odd stage count: unroll 2*NSTG steps so the accumulators return to SA
            for (; t + 3 * NSTG - 1 < ntiles; t += 2 * NSTG)
                static_for<0, 2 * NSTG>([&](auto j) __attribute__((always_inline)) {
                    constexpr int J = decltype(j)::value;
                    constexpr int B = J % NSTG;
                    if constexpr (J % 2 == 0)
                        step(t + J, kbuf<(B + 1) % NSTG>(), kbuf<B>(), vbuf<B>(), vbuf<(B + NSTG - 1) % NSTG>(),
                             SA, SB, Main{}, idlec);
                    else
                        step(t + J, kbuf<(B + 1) % NSTG>(), kbuf<B>(), vbuf<B>(), vbuf<(B + NSTG - 1) % NSTG>(),
                             SB, SA, Main{}, idlec);
                });
        }
        // remaining steps, buffers chosen at run time
        for (; t < ntiles; ++t) {
            const int b = t % NSTG;
            step(t, kbuf_rt((b + 1) % NSTG), kbuf_rt(b), vbuf_rt(b), vbuf_rt((b + NSTG - 1) % NSTG), SA, SB,
                 Tail{}, idlec);
            SA = SB;
        }
    };
    if (idle) run(std::true_type{});
    else run(std::false_type{});

    // normalise and store: lane holds O[qrow][32*db + 8*(j/4) + 4*hf + j%4]
    const uint32_t lb = __float_as_uint(l_run);
    const auto lsw = __builtin_amdgcn_permlane32_swap(lb, lb, false, false);
    const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    const float inv = 1.0f / l_tot;
    if (qrow < N) {
        const int64_t obase = (((int64_t)s * N + qrow) * a.heads + head) * D + 4 * hf;
        if (a.out_fp32) {
            float* o = static_cast<float*>(a.out) + obase;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; j += 4)
                    *reinterpret_cast<float4*>(o + 32 * db + 8 * (j >> 2)) =
                        make_float4(oacc[db][j] * inv, oacc[db][j + 1] * inv,
                                    oacc[db][j + 2] * inv, oacc[db][j + 3] * inv);
        } else {
            uint16_t* o = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; j += 4)
                    *reinterpret_cast<uint2*>(o + 32 * db + 8 * (j >> 2)) =
                        make_uint2(pack_bf16x2(oacc[db][j] * inv, oacc[db][j + 1] * inv),
                                   pack_bf16x2(oacc[db][j + 2] * inv, oacc[db][j + 3] * inv));
        }
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a0, bool fp8, hipStream_t st) {
    AttnArgs a = a0;
    a.qtiles = (a.N + BM - 1) / BM;
    const int64_t blocks = a.nwork;
    if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(NTH);
    if (a.D == 128) {
        if (fp8) hipLaunchKernelGGL((attn_kernel<128, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_kernel<128, false>), grid, block, 0, st, a);
    } else if (a.D == 64) {
        if (fp8) hipLaunchKernelGGL((attn_kernel<64, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_kernel<64, false>), grid, block, 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wf
