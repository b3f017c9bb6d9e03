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

constexpr int kTokTile = 64;                 // tokens per fp8 publish block (one quantisation block)
// tokens per bf16 publish block: 32 gives twice the blocks of 64 and a finer
// last wave of blocks, measured 2-4% faster at the Wan shapes (16 and 128 slower)
constexpr int kTokB = 32;
constexpr int kMaxFramesPerTile = kTokTile + 2;

// Time-axis (cos, sin) table of the frames one publish block (at most 64
// tokens) touches, in dynamic LDS sized per launch: frames_per_tile(HW) rows
// of 32 pairs.
extern __shared__ float2 g_ttab_dyn[];
__host__ __device__ inline int frames_per_tile(int hw) {
    const int f = (kTokTile + hw - 1) / hw + 1;
    return f < kMaxFramesPerTile ? f : kMaxFramesPerTile;
}

__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Projection rows are read exactly once, so their loads take the
// non-temporal path. Page and Q stores stay ordinary: with non-temporal
// stores this kernel measured 7% slower (the attention after it unchanged).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *static_cast<uint4*>(p) = v; }

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

__device__ __forceinline__ void unpack8(uint4 u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Eight input elements as loaded (bf16: one 16-byte vector; fp32: two),
// unpacked to fp32 only when used, so loads can be issued early cheaply.
template <bool IN_FP32>
struct Raw8 {
    uint4 u[IN_FP32 ? 2 : 1];
    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        if constexpr (IN_FP32) {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
            u[0] = p[0];
            u[1] = p[1];
        } else {
            u[0] = ld_stream16(static_cast<const uint16_t*>(base) + elem);
        }
    }
    __device__ __forceinline__ void unpack(float* x) const {
        if constexpr (IN_FP32) {
            const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
        } else {
            unpack8(u[0], x);
        }
    }
};

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

// grid: (ceil(N/32), heads, nslots); block 256. One block rotates and
// publishes 32 tokens of one head of one slot. Reads run along channels
// (coalesced rows of the projection output); page writes run along tokens, so
// K and V are transposed through LDS.
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void publish_bf16_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    float2 (*ttab)[32] = reinterpret_cast<float2 (*)[32]>(g_ttab_dyn);   // time-axis (cos, sin), this tile's frames
    __shared__ __align__(16) uint4 kst[CPR * kTokB];       // K vectors, [ch][tok ^ (ch & 7)]
    __shared__ __align__(16) uint16_t vst[kTokB * D];      // V rows, [tok][d]

    const int tid = threadIdx.x;
    const int sr = blockIdx.z;
    const int s = a.slot_first + sr;
    const int head = blockIdx.y;
    const int n0 = blockIdx.x * kTokB;
    const int p = a.T - 1 - s;                       // context position of slot s
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int n_hi = min(n0 + kTokB, a.N) - 1;
    const int nf = n_hi / HW - f_lo + 1;
    const int hp = a.dt >> 1;

    const int64_t row0 = (int64_t)sr * a.N;
    const int64_t col = (int64_t)head * D;
    auto rotate_and_stage = [&](int tk, int ch, float (&x)[8], float (&y)[8], float (&z)[8]) {
        // x = K, y = Q, z = V of token n0 + tk, channels ch*8 .. ch*8+7
        const int n = n0 + tk;
        const int f = n / HW;
        const int yy = (n / a.frame_w) % a.frame_h;
        const int xw = n % a.frame_w;
        const float2* tf = ttab[f - f_lo];
        const float2* hrow = a.htab + yy * (a.dh >> 1);
        const float2* wrow = a.wtab + xw * (a.dw >> 1);
        rope8(x, ch * 8, tf, hrow, wrow, a.dt, a.dh);
        kst[ch * kTokB + (tk ^ (ch & 7))] = pack8(x);
        if (a.q) {
            rope8(y, ch * 8, tf, hrow, wrow, a.dt, a.dh);
            uint16_t* qp = static_cast<uint16_t*>(a.q_out) + (((int64_t)s * a.heads + head) * a.N + n) * D + ch * 8;
            st16(qp, pack8(y));
        }
        *reinterpret_cast<uint4*>(&vst[tk * D + ch * 8]) = pack8(z);
    };

    if constexpr (!IN_FP32) {
        // Every load of this thread's rows is issued before the time-axis
        // table is built, so the HBM latency overlaps the fp64 sincos work.
        constexpr int IT = (kTokB * CPR + 255) / 256;   // the last may reach past the block
        uint4 kr[IT], qr[IT], vr[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int c = tid + 256 * i, tk = c / CPR, ch = c - tk * CPR;
            const int n = min(n0 + tk, a.N - 1);          // rows past the chunk are read but not used
            const int64_t e = (row0 + n) * a.row_stride + col + ch * 8;
            kr[i] = ld_stream16(static_cast<const uint16_t*>(a.k) + e);
            vr[i] = ld_stream16(static_cast<const uint16_t*>(a.v) + e);
            qr[i] = a.q ? ld_stream16(static_cast<const uint16_t*>(a.q) + e) : make_uint4(0, 0, 0, 0);
        }
        // time-axis angles in fp64: positions grow with the stream
        for (int i = tid; i < nf * hp; i += 256) {
            const int fi = i / hp, m = i - fi * hp;
            const double phi = (double)(slot_t0(a, sr) + f_lo + fi) * a.omega_t[m];
            double sn, cs;
            sincos(phi, &sn, &cs);
            ttab[fi][m] = make_float2((float)cs, (float)sn);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int c = tid + 256 * i, tk = c / CPR, ch = c - tk * CPR;
            if (tk >= kTokB || n0 + tk >= a.N) continue;
            float x[8], y[8], z[8];
            unpack8(kr[i], x);
            unpack8(qr[i], y);
            unpack8(vr[i], z);
            rotate_and_stage(tk, ch, x, y, z);
        }
    } else {
        for (int i = tid; i < nf * hp; i += 256) {
            const int fi = i / hp, m = i - fi * hp;
            const double phi = (double)(slot_t0(a, sr) + f_lo + fi) * a.omega_t[m];
            double sn, cs;
            sincos(phi, &sn, &cs);
            ttab[fi][m] = make_float2((float)cs, (float)sn);
        }
        __syncthreads();
        for (int c = tid; c < kTokB * CPR; c += 256) {
            const int tk = c / CPR, ch = c - tk * CPR;
            if (n0 + tk >= a.N) continue;
            const int64_t e = (row0 + n0 + tk) * a.row_stride + col + ch * 8;
            float x[8], y[8], z[8];
            load8<true>(a.k, e, x);
            if (a.q) load8<true>(a.q, e, y);
            load8<true>(a.v, e, z);
            rotate_and_stage(tk, ch, x, y, z);
        }
    }
    __syncthreads();

    // K pages: one 16-byte vector (8 channels of one token) per thread, tokens fastest
    for (int j = tid; j < CPR * kTokB; j += 256) {
        const int ch = j / kTokB, tk = j - ch * kTokB;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int pg = n / a.pt, tok = n - pg * a.pt;
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + head) * a.pt * D;
        st16(static_cast<uint16_t*>(a.kpage) + k_elem(base, a.pt, tok, ch * 8),
                    kst[ch * kTokB + (tk ^ (ch & 7))]);
    }
    // V pages: one vector of 8 consecutive tokens of one channel per thread,
    // channels fastest. N and pages are multiples of 8, so a group never
    // straddles a page.
    for (int j = tid; j < (kTokB / 8) * D; j += 256) {
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
        st16(a.vpage + v_elem(base, D, tok, d), make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 publish. Q and K are quantised per 64-token block of their chunk
// (blocks restart at each chunk start, so a publish block is exactly one
// quantisation block): scale = absmax / 448, codes = RNE(x / scale) clamped to
// +-448. K first has its chunk's per-channel mean removed; attention adds the
// mean back exactly as q . mean. V stays bf16. Three launches, all with fixed
// summation orders: per-block partial sums of RoPE'd K, their reduction to the
// chunk mean, then the quantising publish.

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    // v_cvt_pk_fp8_f32 rounds to nearest even but turns out-of-range values
    // into NaN, so clamp to the largest finite e4m3 value first
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    c = fminf(fmaxf(c, -448.f), 448.f);
    d = fminf(fmaxf(d, -448.f), 448.f);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, 0, false) & 0xFFFFu;
    return lo | (hi << 16);
}

// Fill the time-axis (cos, sin) table for the frames of one 64-token block.
__device__ __forceinline__ void fill_ttab(float2 (*ttab)[32], const PublishArgs& a, int sr, int f_lo,
                                          int nf) {
    const int hp = a.dt >> 1;
    for (int i = threadIdx.x; i < nf * hp; i += 256) {
        const int fi = i / hp, m = i - fi * hp;
        const double phi = (double)(slot_t0(a, sr) + f_lo + fi) * a.omega_t[m];
        double sn, cs;
        sincos(phi, &sn, &cs);
        ttab[fi][m] = make_float2((float)cs, (float)sn);
    }
}

// grid (ceil(N/64), heads, nslots): per 64-token block, the per-channel sum of
// RoPE'd K over its valid tokens -> kpart[group][head][block][D].
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void kmean_partial_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;
    constexpr int ROWS = 256 / CPR;                  // token lanes per channel vector
    float2 (*ttab)[32] = reinterpret_cast<float2 (*)[32]>(g_ttab_dyn);
    __shared__ float part[ROWS][D];
    const int tid = threadIdx.x;
    const int sr = blockIdx.z, s = a.slot_first + sr, head = blockIdx.y, n0 = blockIdx.x * kTokTile;
    const int p = a.T - 1 - s;
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int nf = (min(n0 + kTokTile, a.N) - 1) / HW - f_lo + 1;
    const int ch = tid % CPR, row = tid / CPR;
    constexpr int IT = kTokTile / ROWS;
    // rows of this thread, loaded before the time table is built (rows past
    // the chunk are clamped to its last row and not summed)
    Raw8<IN_FP32> kin[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int n = min(n0 + row + ROWS * i, a.N - 1);
        kin[i].load(a.k, ((int64_t)sr * a.N + n) * a.row_stride + (int64_t)head * D + ch * 8);
    }
    fill_ttab(ttab, a, sr, f_lo, nf);
    __syncthreads();
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int n = n0 + row + ROWS * i;
        if (n >= a.N) break;
        const int y = (n / a.frame_w) % a.frame_h, xw = n % a.frame_w;
        float x[8];
        kin[i].unpack(x);
        rope8(x, ch * 8, ttab[n / HW - f_lo], a.htab + y * (a.dh >> 1), a.wtab + xw * (a.dw >> 1), a.dt, a.dh);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[row][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
        for (int r = 0; r < ROWS; ++r) sum += part[r][tid];
        const int g = a.table[p * a.ppc] / a.ppc;
        a.kpart[(((int64_t)g * a.heads + head) * a.nblk + blockIdx.x) * D + tid] = sum;
    }
}

// grid (heads, nslots), block D: kmean[group][head][d] = sum of the chunk's
// block partials (fixed order) / N.
template <int D>
__global__ void kmean_reduce_kernel(PublishArgs a) {
    const int s = a.slot_first + blockIdx.y, head = blockIdx.x, d = threadIdx.x;
    const int g = a.table[(a.T - 1 - s) * a.ppc] / a.ppc;
    const float* src = a.kpart + ((int64_t)g * a.heads + head) * a.nblk * D + d;
    // eight loads in flight per iteration, summed in block order
    float sum = 0.f;
    int b = 0;
    for (; b + 8 <= a.nblk; b += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(b + u) * D];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; b < a.nblk; ++b) sum += src[(int64_t)b * D];
    a.kmean[((int64_t)g * a.heads + head) * D + d] = sum / (float)a.N;
}

// grid (ceil(N/64), heads, nslots): quantise and publish one 64-token block.
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void publish_fp8_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    constexpr int ITEMS = kTokTile * CPR / 256;
    constexpr int C16 = D / 16;                      // 16-byte code vectors per token row
    float2 (*ttab)[32] = reinterpret_cast<float2 (*)[32]>(g_ttab_dyn);
    __shared__ float mu[D];
    __shared__ float red[2][4];
    __shared__ __align__(16) uint8_t kcodes[kTokTile * D];   // [tok][16-byte vector ^ (tok % C16)]
    __shared__ __align__(16) uint16_t vst[kTokTile * D];     // V rows, [tok][d]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sr = blockIdx.z, s = a.slot_first + sr, head = blockIdx.y, n0 = blockIdx.x * kTokTile;
    const int p = a.T - 1 - s;
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int nf = (min(n0 + kTokTile, a.N) - 1) / HW - f_lo + 1;
    const int64_t row0 = (int64_t)sr * a.N;
    const int64_t col = (int64_t)head * D;
    // K and V rows of this thread are loaded before the tables are built
    // (rows past the chunk are clamped to its last row and not used)
    Raw8<IN_FP32> kin[ITEMS], qin[ITEMS], vin[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int c = tid + 256 * i;
        const int tk = c / CPR, ch = c - tk * CPR;
        const int64_t e0 = (row0 + min(n0 + tk, a.N - 1)) * a.row_stride + col + ch * 8;
        kin[i].load(a.k, e0);
        vin[i].load(a.v, e0);
        if (a.q) qin[i].load(a.q, e0);
    }
    fill_ttab(ttab, a, sr, f_lo, nf);
    const int g = a.table[p * a.ppc] / a.ppc;
    if (tid < D) mu[tid] = a.kmean[((int64_t)g * a.heads + head) * D + tid];
    __syncthreads();

    float kx[ITEMS][8], qx[ITEMS][8];
    float kmax = 0.f, qmax = 0.f;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int c = tid + 256 * i;
        const int tk = c / CPR, ch = c - tk * CPR;
        const int n = n0 + tk;
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[i][e] = qx[i][e] = 0.f;
        if (n >= a.N) continue;
        kin[i].unpack(kx[i]);
        const int y = (n / a.frame_w) % a.frame_h, xw = n % a.frame_w;
        const float2* tf = ttab[n / HW - f_lo];
        const float2* hrow = a.htab + y * (a.dh >> 1);
        const float2* wrow = a.wtab + xw * (a.dw >> 1);
        rope8(kx[i], ch * 8, tf, hrow, wrow, a.dt, a.dh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kx[i][e] -= mu[ch * 8 + e];
            kmax = fmaxf(kmax, fabsf(kx[i][e]));
        }
        if (a.q) {
            qin[i].unpack(qx[i]);
            rope8(qx[i], ch * 8, tf, hrow, wrow, a.dt, a.dh);
#pragma unroll
            for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(qx[i][e]));
        }
        float vx[8];
        vin[i].unpack(vx);
        *reinterpret_cast<uint4*>(&vst[tk * D + ch * 8]) = pack8(vx);
    }
    kmax = wave_max(kmax);
    qmax = wave_max(qmax);
    if (lane == 0) {
        red[0][wave] = kmax;
        red[1][wave] = qmax;
    }
    __syncthreads();
    kmax = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    qmax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const float ks = kmax > 0.f ? kmax / 448.f : 1.f;     // per-block scales (IEEE divide)
    const float qs = qmax > 0.f ? qmax / 448.f : 1.f;
    const float kinv = 1.f / ks, qinv = 1.f / qs;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int c = tid + 256 * i;
        const int tk = c / CPR, ch = c - tk * CPR;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int v16 = ch >> 1;                     // 16-byte vector of this 8-channel group
        uint2 kc = make_uint2(fp8x4(kx[i][0] * kinv, kx[i][1] * kinv, kx[i][2] * kinv, kx[i][3] * kinv),
                              fp8x4(kx[i][4] * kinv, kx[i][5] * kinv, kx[i][6] * kinv, kx[i][7] * kinv));
        *reinterpret_cast<uint2*>(&kcodes[(tk * C16 + (v16 ^ (tk % C16))) * 16 + (ch & 1) * 8]) = kc;
        if (a.q) {
            uint2 qc = make_uint2(fp8x4(qx[i][0] * qinv, qx[i][1] * qinv, qx[i][2] * qinv, qx[i][3] * qinv),
                                  fp8x4(qx[i][4] * qinv, qx[i][5] * qinv, qx[i][6] * qinv, qx[i][7] * qinv));
            uint8_t* qp = static_cast<uint8_t*>(a.q_out) + (((int64_t)s * a.heads + head) * a.N + n) * D + ch * 8;
            *reinterpret_cast<uint2*>(qp) = qc;
        }
    }
    if (a.q && tid == 0) a.q_scales[((int64_t)s * a.heads + head) * a.nblk + blockIdx.x] = qs;
    __syncthreads();

    // K code pages: one 16-byte vector (16 channels of one token) per thread, tokens fastest
    for (int j = tid; j < C16 * kTokTile; j += 256) {
        const int v16 = j / kTokTile, tk = j - v16 * kTokTile;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int pg = n / a.pt, tok = n - pg * a.pt;
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + head) * a.pt * D;
        st16(static_cast<uint8_t*>(a.kpage) + k8_byte(base, a.pt, tok, v16 * 16),
                    *reinterpret_cast<const uint4*>(&kcodes[(tk * C16 + (v16 ^ (tk % C16))) * 16]));
    }
    if (tid < kTokTile && n0 + tid < a.N) {
        const int n = n0 + tid;
        const int pg = n / a.pt, tok = n - pg * a.pt;
        const int phys = a.table[p * a.ppc + pg];
        a.kscale[((int64_t)phys * a.heads + head) * a.pt + tok] = ks;
    }
    // V pages as in the bf16 publish
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
        st16(a.vpage + v_elem(base, D, tok, d), make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// table[p][i] = group(p) * ppc + i; group(p) = p for the anchor, otherwise
// A + ((p - A + ring) mod (T - A)); while the store holds an anchor chunk
// (store_anchor >= 0, pipeline fill) the store position writes that anchor's
// group.
// One block. With a device round counter the ring offset is read from it
// (the next round's) and written back once every thread has read it, so the
// same launch advances the pool whichever round it runs in.
__global__ __launch_bounds__(1024) void page_table_kernel(int32_t* table, int T, int A, int ppc, int64_t ring,
                                                          int64_t* ring_dev, int store_pos, int store_anchor) {
    if (ring_dev) ring = ring_dev[0] + 1;
    const int R = T - A;
    for (int i = threadIdx.x; i < T * ppc; i += blockDim.x) {
        const int p = i / ppc, pg = i - p * ppc;
        int g = p < A ? p : A + (int)(((int64_t)(p - A) + ring) % R);
        if (p == store_pos && store_anchor >= 0) g = store_anchor;
        table[i] = g * ppc + pg;
    }
    if (ring_dev) {
        __syncthreads();
        if (threadIdx.x == 0) ring_dev[0] = ring;
    }
}

}  // namespace

hipError_t launch_page_table(int32_t* table, int T, int A, int ppc, int64_t ring, int64_t* ring_dev, int store_pos,
                             int store_anchor, hipStream_t st) {
    const int n = T * ppc;
    const int threads = n < 1024 ? (n + 63) / 64 * 64 : 1024;
    hipLaunchKernelGGL(page_table_kernel, dim3(1), dim3(threads), 0, st, table, T, A, ppc, ring, ring_dev,
                       store_pos, store_anchor);
    return hipGetLastError();
}

template <int D, bool IN_FP32>
hipError_t launch_publish_t(const PublishArgs& a, bool fp8, hipStream_t st) {
    const dim3 grid((a.N + kTokTile - 1) / kTokTile, a.heads, a.nslots);
    const size_t tbytes = (size_t)frames_per_tile(a.frame_h * a.frame_w) * 32 * sizeof(float2);
    if (!fp8) {
        const dim3 gb((a.N + kTokB - 1) / kTokB, a.heads, a.nslots);
        hipLaunchKernelGGL((publish_bf16_kernel<D, IN_FP32>), gb, dim3(256), tbytes, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((kmean_partial_kernel<D, IN_FP32>), grid, dim3(256), tbytes, st, a);
    hipLaunchKernelGGL((kmean_reduce_kernel<D>), dim3(a.heads, a.nslots), dim3(D), 0, st, a);
    hipLaunchKernelGGL((publish_fp8_kernel<D, IN_FP32>), grid, dim3(256), tbytes, st, a);
    return hipGetLastError();
}

hipError_t launch_publish(const PublishArgs& a, bool fp8, hipStream_t st) {
    if (a.D == 128) return a.in_fp32 ? launch_publish_t<128, true>(a, fp8, st) : launch_publish_t<128, false>(a, fp8, st);
    if (a.D == 64) return a.in_fp32 ? launch_publish_t<64, true>(a, fp8, st) : launch_publish_t<64, false>(a, fp8, st);
    return hipErrorInvalidValue;
}

}  // namespace wf
