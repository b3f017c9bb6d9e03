// QKV projection with RoPE and publish as its epilogue, gfx950: bf16 MFMA, or
// fp8 e4m3 MFMA for W8A8 operands.
//
// The pages publish K/V right after the QKV projection and RoPE (Wave
// Forcing, hyper.ai summary, section "Method", WaveRT paragraph; e-cogni.com.br,
// "Como funciona"); the projection maps the hidden state (heads x 128 wide,
// thelatestinai.com listing, Table 11) to [Q | K | V]. Here the projection
// output never goes to memory: each workgroup's accumulators are rotated and
// written straight into the Q buffer and the K/V pages of the slot's context
// position, in the same formats the publish kernel writes.
//
//   qkv[n][o] = sum_c x[n][c] * w[o][c] + b[o]      (w in [out][in] layout)
//
// Workgroup tile: 256 tokens of one slot's chunk x 256 output channels. 8
// waves (two per SIMD), each 64 tokens x 128 channels as 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, so every X fragment read from LDS feeds four
// MFMAs and every W fragment two. A wave's 128 channels lie wholly inside Q,
// K or V (h*d is a multiple of 128), so the orientation below is per wave.
//   Q and K tiles compute the transposed block C^T[channel][token], so a lane
//   holds one token and runs of 4 consecutive channels: the RoPE pairs
//   (2m, 2m+1) are in-lane, and a lane pair (l, l+32) holds 8 consecutive
//   channels, i.e. one 16-byte K page vector.
//   V tiles compute C[token][channel], so a lane holds one channel and runs of
//   4 consecutive tokens: a lane pair holds 8 consecutive tokens of one
//   channel, i.e. one 16-byte V page vector.
// Both orientations read the same LDS fragments (16 bytes = 8 consecutive
// hidden channels of one row of x or w) and only swap the MFMA operands.
//
// Operands arrive by LDS DMA in stages of 128 bytes per row (64 bf16 or 128
// e4m3 hidden channels), double-buffered. 16-byte vector kv of row r sits in
// slot kv ^ ((r >> 1) & 7), so that each DMA instruction reads eight whole
// rows (eight 128-byte lines of x or w) and the fragment reads of 16 lanes (16
// consecutive rows, one kv) fall on 16 distinct 16-byte bank groups.
//
// W8A8 (the pages pair 8-bit weights and activations with the quantised
// attention: e-cogni.com.br, "Como funciona"; thelatestinai.com listing,
// Table 6): x and w hold e4m3 codes with one fp32 scale per row of each
// (per token, per output channel). The stage layout and DMA are the same
// bytes; each lane feeds v_mfma_f32_32x32x64_f8f6f4 with 32 consecutive codes
// (two 16-byte vectors), and the epilogue multiplies every accumulator by its
// token's and channel's scales before the bias. Unlike the bf16 MFMA, whose
// fp32 sums of bf16 products round like ordinary fp32 additions, the e4m3 MFMA
// keeps each instruction's 64 products only to a fixed distance below its
// largest one: a sum of codes can lose up to about 2^-12 of sum |x w| (the
// W8A8 parity bound allows twice that).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int PM = kProjTokens;   // tokens per workgroup tile
constexpr int PC = kProjChannels; // output channels per workgroup tile
constexpr int BK = 64;            // bf16 hidden channels per stage (128 bytes per row)
constexpr int PNT = 512;          // threads per workgroup (8 waves)
constexpr int XI = PM / 8 / 8;    // x DMA instructions per wave per stage (8 rows each)
constexpr int WI = PC / 8 / 8;    // w DMA instructions per wave per stage
// Buffer offset past every region (each is under 2^31 bytes): loads zeros.
// The per-stage addend is below 2^31 too, so kOOB plus it stays out of range.
constexpr uint32_t kOOB = 0x80000000u;

__shared__ __align__(16) uint16_t g_px0[PM * BK];
__shared__ __align__(16) uint16_t g_px1[PM * BK];
__shared__ __align__(16) uint16_t g_pw0[PC * BK];
__shared__ __align__(16) uint16_t g_pw1[PC * BK];
// row- and column-axis (cos, sin) tables: [frame_h][dh/2] then [frame_w][dw/2]
__shared__ float2 g_prtab[kProjMaxRopeEntries];
// time-axis (cos, sin) of every frame the tile touches: [frame][32]
__shared__ float2 g_pttab[kProjMaxFrames * 32];

template <int I>
__device__ __forceinline__ uint16_t* xbuf() {
    if constexpr (I == 0) return g_px0;
    else return g_px1;
}
template <int I>
__device__ __forceinline__ uint16_t* wbuf() {
    if constexpr (I == 0) return g_pw0;
    else return g_pw1;
}

template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// All LDS DMA of the stage about to be read has landed in every wave (each
// wave waited for its own before): a bare barrier orders the buffers.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef int i32x4 __attribute__((ext_vector_type(4)));
// Buffer resource for raw loads from [base, base + bytes).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int32_t bytes) {
    const uint64_t b = (uint64_t)base;
    i32x4 r;
    r.x = (int)(uint32_t)b;
    r.y = (int)(uint32_t)(b >> 32) & 0xFFFF;    // stride 0
    r.z = bytes;
    r.w = 0x00020000;
    return r;
}
// LDS DMA of 16 bytes per lane to LDS address lds + 16 * lane. Written as
// inline asm: it writes LDS, not registers, and the kernel orders every read
// of a stage after that stage's DMA with an explicit vmcnt wait and a barrier,
// so the compiler must not add waits of its own before the fragment reads
// that follow the next stage's DMA (it cannot tell the two buffers apart).
__device__ __forceinline__ void dma16(i32x4 r, const void* lds, uint32_t voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m), "v"(voff), "s"(r) : "memory", "m0");
}

// byte offset of 16-byte vector kv of row r inside a stage
__device__ __forceinline__ int swz(int r, int kv) { return r * 128 + ((kv ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ i32x8 as_i32x8(uint4 a, uint4 b) {
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int D, bool F8>
__global__ __launch_bounds__(PNT, 1) void proj_publish_kernel(ProjArgs a) {
    constexpr int ESZ = F8 ? 1 : 2;               // bytes per operand element
    constexpr int BKE = 128 / ESZ;                // hidden channels per stage
    // ---- which tile: XCD x takes a block of (token-tile rows x channel tiles)
    const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int cg = xcd % a.g_ct, mg = xcd / a.g_ct;
    const int c_lo = cg * a.ctiles / a.g_ct, c_hi = (cg + 1) * a.ctiles / a.g_ct;
    const int r_lo = mg * a.mrows / a.g_mt, r_hi = (mg + 1) * a.mrows / a.g_mt;
    const int nc = c_hi - c_lo;
    if (nc <= 0) return;
    const int row = r_lo + j / nc;
    if (row >= r_hi) return;                       // padding of the per-XCD ranges
    const int ct = c_lo + j % nc;
    const int sr = row / a.mtiles, mt = row - sr * a.mtiles;
    const int s = a.slot_first + sr;
    const int N = a.N, hd = a.heads * D;
    const int n0 = mt * PM;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int wm = wave & 3, wc = wave >> 2;       // 64-token and 128-channel block of this wave
    const int ob = ct * PC + wc * 128;             // first output channel of this wave
    const bool live = ob < 3 * hd;                 // the last tile may reach past 3*h*d
    const int kind = live ? ob / hd : 0;           // 0 Q, 1 K, 2 V (uniform: h*d % 128 == 0)
    const bool rope = live && kind < 2;
    const bool tile_rope = ct * PC < 2 * hd;       // some wave of the tile rotates

    const i32x4 xrs = make_rsrc(a.x, a.xbytes);
    const i32x4 wrs = make_rsrc(a.w, a.wbytes);

    // ---- RoPE tables: the time-axis frequency of this thread's table entry
    // and the row/column (cos, sin) tables, loaded and waited for before any
    // DMA, so the DMA wait counts stay exact; the fp64 sincos runs while the
    // first stage is in flight
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int nf = (min(n0 + PM, N) - 1) / HW - f_lo + 1;
    const int hp = a.dt >> 1;
    static_assert(kProjMaxFrames * 32 <= PNT, "one time-table entry per thread");
    const bool tt = tile_rope && tid < nf * hp;
    const double om = tt ? a.omega_t[tid % hp] : 0.0;
    const int nh = a.frame_h * (a.dh >> 1), nrope = nh + a.frame_w * (a.dw >> 1);
    constexpr int RE = kProjMaxRopeEntries / PNT;
    float2 rt[RE];
#pragma unroll
    for (int e = 0; e < RE; ++e) {
        const int idx = tid + e * PNT;
        rt[e] = (tile_rope && idx < nrope) ? (idx < nh ? a.htab[idx] : a.wtab[idx - nh]) : make_float2(0.f, 0.f);
    }
    wait_vmem_n<0>();
#pragma unroll
    for (int e = 0; e < RE; ++e) {
        const int idx = tid + e * PNT;
        if (tile_rope && idx < nrope) g_prtab[idx] = rt[e];
    }

    // ---- DMA offsets: lane covers vector (lane % 8) of row (lane / 8) of each
    // 8-row instruction; the vector it fetches is the one that slot holds
    uint32_t xoff[XI], woff[WI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = (wave * XI + i) * 8 + (lane >> 3);
        const int kv = (lane & 7) ^ ((r >> 1) & 7);
        const int n = n0 + r;
        xoff[i] = n < N ? (uint32_t)(((int64_t)sr * N + n) * a.x_stride * ESZ + kv * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int r = (wave * WI + i) * 8 + (lane >> 3);
        const int kv = (lane & 7) ^ ((r >> 1) & 7);
        const int o = ct * PC + r;
        woff[i] = o < 3 * hd ? (uint32_t)((int64_t)o * a.hidden * ESZ + kv * 16) : kOOB;
    }
    auto dma_stage = [&](auto I, int kt) {
        constexpr int B = decltype(I)::value;
        const uint32_t kb = (uint32_t)kt * 128;
        uint8_t* xl = reinterpret_cast<uint8_t*>(xbuf<B>());
        uint8_t* wl = reinterpret_cast<uint8_t*>(wbuf<B>());
#pragma unroll
        for (int i = 0; i < XI; ++i) dma16(xrs, xl + (wave * XI + i) * 1024, xoff[i] + kb);
#pragma unroll
        for (int i = 0; i < WI; ++i) dma16(wrs, wl + (wave * WI + i) * 1024, woff[i] + kb);
    };
    const int nk = a.hidden / BKE;
    dma_stage(std::integral_constant<int, 0>{}, 0);

    if (tt) {
        const int fi = tid / hp, m = tid - fi * hp;
        double sn, cs;
        sincos((double)(slot_t0(a, sr) + f_lo + fi) * om, &sn, &cs);
        g_pttab[fi * 32 + m] = make_float2((float)cs, (float)sn);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.f;

    // One stage: wait for its DMA and the barrier, read every fragment of the
    // stage (the reads of the second half after the next stage's DMA into the
    // other buffer, which every wave finished reading before this barrier),
    // then 32 MFMAs, which the next stage's DMA lands behind.
    // TR: the transposed block C^T[channel][token] (Q and K waves).
    auto stage = [&](auto I, auto TR, int kt) {
        constexpr int B = decltype(I)::value;
        wait_vmem_n<0>();
        stage_barrier();
        const uint8_t* xl = reinterpret_cast<const uint8_t*>(xbuf<B>());
        const uint8_t* wl = reinterpret_cast<const uint8_t*>(wbuf<B>());
        if constexpr (F8) {
            // two 64-code K steps; lane half hf supplies codes 32 hf .. 32 hf + 31
            // of each, i.e. vectors 4 ks + 2 hf and 4 ks + 2 hf + 1 of its row
            uint4 xf8[2][2][2], wf8[2][4][2];
            auto rd8 = [&](int ks) {
                const int kv = 4 * ks + 2 * hf;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        xf8[ks][i][u] = *reinterpret_cast<const uint4*>(xl + swz(wm * 64 + i * 32 + l32, kv + u));
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        wf8[ks][jj][u] = *reinterpret_cast<const uint4*>(wl + swz(wc * 128 + jj * 32 + l32, kv + u));
            };
            rd8(0);
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) dma_stage(std::integral_constant<int, B ^ 1>{}, kt + 1);
            __builtin_amdgcn_sched_barrier(0);
            rd8(1);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const i32x8 xa = as_i32x8(xf8[ks][i][0], xf8[ks][i][1]);
                        const i32x8 wa = as_i32x8(wf8[ks][jj][0], wf8[ks][jj][1]);
                        if constexpr (decltype(TR)::value)
                            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, xa, acc[i][jj],
                                                                                        0, 0, 0, 0, 0, 0);
                        else
                            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, wa, acc[i][jj],
                                                                                        0, 0, 0, 0, 0, 0);
                    }
            return;
        }
        bf16x8 xf[BK / 16][2], wf_[BK / 16][4];
        auto rd = [&](int ks) {
            const int kv = ks * 2 + hf;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                xf[ks][i] = *reinterpret_cast<const bf16x8*>(xl + swz(wm * 64 + i * 32 + l32, kv));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                wf_[ks][jj] = *reinterpret_cast<const bf16x8*>(wl + swz(wc * 128 + jj * 32 + l32, kv));
        };
        rd(0);
        rd(1);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) dma_stage(std::integral_constant<int, B ^ 1>{}, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        rd(2);
        rd(3);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if constexpr (decltype(TR)::value)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf_[ks][jj], xf[ks][i], acc[i][jj], 0, 0, 0);
                    else
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[ks][i], wf_[ks][jj], acc[i][jj], 0, 0, 0);
                }
    };
    // every wave runs the same stages (and barriers) whichever orientation it takes
    auto kloop = [&](auto TR) {
        for (int kt = 0; kt < nk; kt += 2) {
            stage(std::integral_constant<int, 0>{}, TR, kt);
            if (kt + 1 < nk) stage(std::integral_constant<int, 1>{}, TR, kt + 1);
        }
    };
    if (rope || !live) kloop(std::true_type{});
    else kloop(std::false_type{});
    __syncthreads();                               // stage buffers free, time table visible
    if (!live) return;

    // ---- epilogue: (e4m3: token and channel scales,) bias, RoPE (Q, K), bf16,
    // then out to the Q buffer / pages,
    // in two passes of 64 channels. Each wave stages a 64 x 64 bf16 block in
    // LDS in the destination's order and writes it out with 16-byte stores:
    // 1 KB contiguous per K or V instruction, 128-byte row pieces for Q.
    const int p = a.T - 1 - s;                     // context position of slot s
    const int pt = a.pt;
    uint8_t* st = reinterpret_cast<uint8_t*>(wave < 4 ? g_px0 : g_px1) + (wave & 3) * 8192;
    const int tb = n0 + wm * 64;                   // first token of this wave
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int oc = ob + 64 * h2;               // first output channel of this pass
        if (rope) {
            const int cb = oc - kind * hd;         // its channel inside Q or K
            // [token 64][8 x 16-byte chunks of 8 channels], chunk slot c ^ (t & 7)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int t = i * 32 + l32;
                const int n = min(tb + t, N - 1);
                const float sxt = F8 ? a.xs[(int64_t)sr * N + n] : 1.f;
                const int f = n / HW - f_lo;
                const int yy = (n / a.frame_w) % a.frame_h;
                const int xw = n % a.frame_w;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int cl = jj * 32 + 8 * g + 4 * hf;            // 4 consecutive channels
                        const int d0 = (cb + cl) % D;
                        const uint2 bq = a.bias ? *reinterpret_cast<const uint2*>(a.bias + oc + cl) : make_uint2(0, 0);
                        const f32x16& A = acc[i][2 * h2 + jj];
                        float v[4] = {A[4 * g + 0], A[4 * g + 1], A[4 * g + 2], A[4 * g + 3]};
                        if constexpr (F8) {
                            const float4 sw = *reinterpret_cast<const float4*>(a.ws + oc + cl);
                            v[0] = v[0] * sxt * sw.x;
                            v[1] = v[1] * sxt * sw.y;
                            v[2] = v[2] * sxt * sw.z;
                            v[3] = v[3] * sxt * sw.w;
                        }
                        v[0] += __uint_as_float(bq.x << 16);
                        v[1] += __uint_as_float(bq.x & 0xFFFF0000u);
                        v[2] += __uint_as_float(bq.y << 16);
                        v[3] += __uint_as_float(bq.y & 0xFFFF0000u);
#pragma unroll
                        for (int pr = 0; pr < 2; ++pr) {
                            const int dc = d0 + 2 * pr;
                            float2 c2;
                            if (dc < a.dt) c2 = g_pttab[f * 32 + (dc >> 1)];
                            else if (dc < a.dt + a.dh) c2 = g_prtab[yy * (a.dh >> 1) + ((dc - a.dt) >> 1)];
                            else c2 = g_prtab[nh + xw * (a.dw >> 1) + ((dc - a.dt - a.dh) >> 1)];
                            const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
                            v[2 * pr] = fmaf(x0, c2.x, -x1 * c2.y);
                            v[2 * pr + 1] = fmaf(x0, c2.y, x1 * c2.x);
                        }
                        const int chunk = jj * 4 + g;
                        *reinterpret_cast<uint2*>(st + t * 128 + ((chunk ^ (t & 7)) << 4) + hf * 8) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
            }
            if (kind == 0) {
                // Q [s][head][n][D]: 8 lanes per token write its 64 channels (128 bytes)
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const int t = it * 8 + (lane >> 3), chunk = lane & 7;
                    const uint4 val = *reinterpret_cast<const uint4*>(st + t * 128 + ((chunk ^ (t & 7)) << 4));
                    const int n = tb + t;
                    if (n >= N) continue;
                    const int c = cb + chunk * 8;
                    const int head = c / D, d = c - head * D;
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.q_out) +
                                              (((int64_t)s * a.heads + head) * N + n) * D + d) = val;
                }
            } else {
                // K pages [phys][head][D/8][pt][8]: one lane per token, one 8-channel vector per store
                const int n = tb + lane;
                const int tok = n % pt;
                const int64_t phys = a.table[p * a.ppc + min(n, N - 1) / pt];
#pragma unroll
                for (int v8 = 0; v8 < 8; ++v8) {
                    const uint4 val = *reinterpret_cast<const uint4*>(st + lane * 128 + ((v8 ^ (lane & 7)) << 4));
                    if (n >= N) continue;
                    const int c = cb + v8 * 8;
                    const int head = c / D, d = c - head * D;
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.kpage) + (phys * a.heads + head) * pt * D +
                                              ((int64_t)(d >> 3) * pt + tok) * 8) = val;
                }
            }
        } else {
            const int cb = oc - 2 * hd;            // first channel of this pass inside V
            // [channel 64][8 x 16-byte chunks of 8 tokens], chunk slot tg ^ (c & 7)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int c = jj * 32 + l32;
                const float bb = a.bias ? bf_to_f(a.bias[oc + c]) : 0.f;
                const float swc = F8 ? a.ws[oc + c] : 1.f;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& Ai = acc[i][2 * h2 + jj];
                        const int chunk = i * 4 + g;                        // tokens 8*chunk + 4*hf .. +3
                        float v[4] = {Ai[4 * g], Ai[4 * g + 1], Ai[4 * g + 2], Ai[4 * g + 3]};
                        if constexpr (F8) {
                            // N is a multiple of 8: these 4 tokens are all inside the chunk or all past it
                            const int n4 = min(tb + 8 * chunk + 4 * hf, N - 4);
                            const float4 sx = *reinterpret_cast<const float4*>(a.xs + (int64_t)sr * N + n4);
                            v[0] = v[0] * sx.x * swc;
                            v[1] = v[1] * sx.y * swc;
                            v[2] = v[2] * sx.z * swc;
                            v[3] = v[3] * sx.w * swc;
                        }
                        *reinterpret_cast<uint2*>(st + c * 128 + ((chunk ^ (c & 7)) << 4) + hf * 8) =
                            make_uint2(pack_bf16x2(v[0] + bb, v[1] + bb), pack_bf16x2(v[2] + bb, v[3] + bb));
                    }
            }
            // V pages [phys][head][pt/8][D][8]: one lane per channel, one 8-token group per store
            const int c = cb + lane;
            const int head = c / D, d = c - head * D;
#pragma unroll
            for (int tg = 0; tg < 8; ++tg) {
                const uint4 val = *reinterpret_cast<const uint4*>(st + lane * 128 + ((tg ^ (lane & 7)) << 4));
                const int n = tb + tg * 8;
                if (n >= N) continue;              // N is a multiple of 8: all 8 tokens or none
                const int tok = n % pt;
                const int64_t phys = a.table[p * a.ppc + n / pt];
                *reinterpret_cast<uint4*>(a.vpage + (phys * a.heads + head) * pt * D + ((int64_t)(tok >> 3) * D + d) * 8) = val;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-row e4m3 quantisation of W8A8 operands (a token row of the activations,
// an output-channel row of the weights). One wave per row, held in registers:
// the row's absmax is reduced across the wave, scale = absmax / 448 (IEEE
// divide; 1 for an all-zero row), and every code is decided on the IEEE fp32
// quotient x / scale, rounded to nearest even and saturated at +-448. QV
// 16-byte vectors per lane hold the row: the smallest of 4, 8, 16 that fits,
// so narrow rows leave registers for more waves in flight.
constexpr int kQuantMaxQV = kQuantMaxCols / 8 / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint32_t code2(float p, float q) {
    // v_cvt_pk_fp8_f32 rounds to nearest even; out-of-range inputs would
    // become NaN, so saturate first
    p = fminf(fmaxf(p, -448.f), 448.f);
    q = fminf(fmaxf(q, -448.f), 448.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p, q, 0, false) & 0xFFFFu;
}

template <int QV>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* x, int64_t rows, int cols,
                                                         int64_t x_stride, uint8_t* codes,
                                                         int64_t code_stride, float* scales) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                       // whole waves
    const int lane = threadIdx.x & 63;
    const int nv = cols >> 3;
    const uint16_t* xr = x + row * x_stride;
    uint4 v[QV];
    uint32_t amax_bits = 0;                        // |bf16| bit patterns order like their values
#pragma unroll
    for (int i = 0; i < QV; ++i) {
        const int vi = lane + 64 * i;
        v[i] = vi < nv ? *reinterpret_cast<const uint4*>(xr + vi * 8) : make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            amax_bits = max(amax_bits, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
    }
    const float amax = wave_max(__uint_as_float(amax_bits << 16));
    const float sc = amax > 0.f ? amax / 448.f : 1.f;
    uint8_t* cr = codes + row * code_stride;
#pragma unroll
    for (int i = 0; i < QV; ++i) {
        const int vi = lane + 64 * i;
        if (vi >= nv) continue;
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c[e] = code2(__uint_as_float(w4[e] << 16) / sc, __uint_as_float(w4[e] & 0xFFFF0000u) / sc);
        *reinterpret_cast<uint2*>(cr + vi * 8) = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
    }
    if (lane == 0) scales[row] = sc;
}

}  // namespace

int proj_frames_per_tile(int hw) { return (PM - 1) / hw + 2; }

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, int64_t x_stride, uint8_t* codes,
                             int64_t code_stride, float* scales, hipStream_t st) {
    const int64_t blocks = (rows + 3) / 4;
    const int per_lane = (cols / 8 + 63) / 64;
    static_assert(kQuantMaxQV == 16, "vectors per lane of the widest row");
    if (per_lane <= 4)
        hipLaunchKernelGGL(quant_rows_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, x_stride,
                           codes, code_stride, scales);
    else if (per_lane <= 8)
        hipLaunchKernelGGL(quant_rows_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, x_stride,
                           codes, code_stride, scales);
    else
        hipLaunchKernelGGL(quant_rows_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, x_stride,
                           codes, code_stride, scales);
    return hipGetLastError();
}

hipError_t launch_project(const ProjArgs& a, bool f8, int nblocks, hipStream_t st) {
    if (a.D == 128 && f8)
        hipLaunchKernelGGL((proj_publish_kernel<128, true>), dim3(nblocks), dim3(PNT), 0, st, a);
    else if (a.D == 128)
        hipLaunchKernelGGL((proj_publish_kernel<128, false>), dim3(nblocks), dim3(PNT), 0, st, a);
    else if (a.D == 64 && f8)
        hipLaunchKernelGGL((proj_publish_kernel<64, true>), dim3(nblocks), dim3(PNT), 0, st, a);
    else if (a.D == 64)
        hipLaunchKernelGGL((proj_publish_kernel<64, false>), dim3(nblocks), dim3(PNT), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wf
