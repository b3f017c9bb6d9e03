// Fused 3D-RoPE + K/V publish into the paged slot pool, and the page-table
// rewrite used by the round advance. gfx950 (CDNA4), wave64.
//
// Publishing follows the WaveRT description (Wave Forcing, hyper.ai summary,
// section "Method"): K/V are published right after QKV projection and RoPE,
// written straight into the ordered attention slots (paged delivery), so the
// attention kernel never concatenates or copies context.
//
// Page formats written here are described in wf_internal.h (16-byte vectors,
// K channel-chunk major, V token-chunk major).
#include <hip/hip_runtime.h>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kTokTile = 64;                 // tokens per publish block
constexpr int kMaxFramesPerTile = kTokTile + 2;

__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

template <bool IN_FP32>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* x) {
    if constexpr (IN_FP32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

__device__ __forceinline__ uint4 pack8(const float* x) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

// Rotate the 4 channel pairs of one 8-channel vector starting at channel c0.
__device__ __forceinline__ void rope8(float* x, int c0, const float2* ttab_f, const float2* hrow,
                                      const float2* wrow, int dt, int dh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = c0 + 2 * i;
        float2 cs;
        if (c < dt) cs = ttab_f[c >> 1];
        else if (c < dt + dh) cs = hrow[(c - dt) >> 1];
        else cs = wrow[(c - dt - dh) >> 1];
        const float a = x[2 * i], b = x[2 * i + 1];
        x[2 * i] = fmaf(a, cs.x, -b * cs.y);
        x[2 * i + 1] = fmaf(a, cs.y, b * cs.x);
    }
}

// grid: (ceil(N/64), heads, nslots); block 256. One block rotates and
// publishes 64 tokens of one head of one slot. Reads run along channels
// (coalesced rows of the projection output); page writes run along tokens, so
// K and V are transposed through LDS.
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void publish_bf16_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    __shared__ float2 ttab[kMaxFramesPerTile][32];   // time-axis (cos, sin), this tile's frames
    __shared__ __align__(16) uint4 kst[CPR * kTokTile];       // K vectors, [ch][tok ^ (ch & 7)]
    __shared__ __align__(16) uint16_t vst[kTokTile * D];      // V rows, [tok][d]

    const int tid = threadIdx.x;
    const int sr = blockIdx.z;
    const int s = a.slot_first + sr;
    const int head = blockIdx.y;
    const int n0 = blockIdx.x * kTokTile;
    const int p = a.T - 1 - s;                       // context position of slot s
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int n_hi = min(n0 + kTokTile, a.N) - 1;
    const int nf = n_hi / HW - f_lo + 1;
    const int hp = a.dt >> 1;

    // time-axis angles in fp64: positions grow with the stream
    for (int i = tid; i < nf * hp; i += 256) {
        const int fi = i / hp, m = i - fi * hp;
        const double phi = (double)(a.t0[sr] + f_lo + fi) * a.omega_t[m];
        double sn, cs;
        sincos(phi, &sn, &cs);
        ttab[fi][m] = make_float2((float)cs, (float)sn);
    }
    __syncthreads();

    const int64_t row0 = (int64_t)sr * a.N;
    const int64_t col = (int64_t)head * D;
    for (int c = tid; c < kTokTile * CPR; c += 256) {
        const int tk = c / CPR, ch = c - tk * CPR;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int f = n / HW;
        const int y = (n / a.frame_w) % a.frame_h;
        const int xw = n % a.frame_w;
        const float2* tf = ttab[f - f_lo];
        const float2* hrow = a.htab + y * (a.dh >> 1);
        const float2* wrow = a.wtab + xw * (a.dw >> 1);
        const int64_t e = (row0 + n) * a.row_stride + col + ch * 8;
        float x[8];
        load8<IN_FP32>(a.k, e, x);
        rope8(x, ch * 8, tf, hrow, wrow, a.dt, a.dh);
        kst[ch * kTokTile + (tk ^ (ch & 7))] = pack8(x);
        if (a.q) {
            load8<IN_FP32>(a.q, e, x);
            rope8(x, ch * 8, tf, hrow, wrow, a.dt, a.dh);
            uint16_t* qp = static_cast<uint16_t*>(a.q_out) +
                           (((int64_t)s * a.heads + head) * a.N + n) * D + ch * 8;
            *reinterpret_cast<uint4*>(qp) = pack8(x);
        }
        load8<IN_FP32>(a.v, e, x);
        *reinterpret_cast<uint4*>(&vst[tk * D + ch * 8]) = pack8(x);
    }
    __syncthreads();

    // K pages: one 16-byte vector (8 channels of one token) per thread, tokens fastest
    for (int j = tid; j < CPR * kTokTile; j += 256) {
        const int ch = j / kTokTile, tk = j - ch * kTokTile;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int pg = n / a.pt, tok = n - pg * a.pt;
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + head) * a.pt * D;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.kpage) + k_elem(base, a.pt, tok, ch * 8)) =
            kst[ch * kTokTile + (tk ^ (ch & 7))];
    }
    // V pages: one vector of 8 consecutive tokens of one channel per thread,
    // channels fastest. N and pages are multiples of 8, so a group never
    // straddles a page.
    for (int j = tid; j < (kTokTile / 8) * D; j += 256) {
        const int kc = j / D, d = j - kc * D;
        const int n = n0 + kc * 8;
        if (n >= a.N) continue;
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w[r] = (uint32_t)vst[(kc * 8 + 2 * r) * D + d] | ((uint32_t)vst[(kc * 8 + 2 * r + 1) * D + d] << 16);
        const int pg = n / a.pt, tok = n - pg * a.pt;
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + head) * a.pt * D;
        *reinterpret_cast<uint4*>(a.vpage + v_elem(base, D, tok, d)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// table[p][i] = group(p) * ppc + i; group(p) = p for the anchor, otherwise
// A + ((p - A + ring) mod (T - A)).
__global__ void page_table_kernel(int32_t* table, int T, int A, int ppc, int64_t ring) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * ppc) return;
    const int p = i / ppc, pg = i - p * ppc;
    const int R = T - A;
    const int g = p < A ? p : A + (int)(((int64_t)(p - A) + ring) % R);
    table[i] = g * ppc + pg;
}

}  // namespace

hipError_t launch_page_table(int32_t* table, int T, int A, int ppc, int64_t ring, hipStream_t st) {
    const int n = T * ppc;
    hipLaunchKernelGGL(page_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, table, T, A, ppc, ring);
    return hipGetLastError();
}

hipError_t launch_publish(const PublishArgs& a, bool fp8, hipStream_t st) {
    if (fp8) return hipErrorNotSupported;
    const dim3 grid((a.N + kTokTile - 1) / kTokTile, a.heads, a.nslots);
    if (a.D == 128) {
        if (a.in_fp32) hipLaunchKernelGGL((publish_bf16_kernel<128, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((publish_bf16_kernel<128, false>), grid, dim3(256), 0, st, a);
    } else if (a.D == 64) {
        if (a.in_fp32) hipLaunchKernelGGL((publish_bf16_kernel<64, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((publish_bf16_kernel<64, false>), grid, dim3(256), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wf
