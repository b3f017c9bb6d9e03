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

#include <mutex>

#include "wf_internal.h"

// Scratch of wf_kv_publish_noalloc: the fp8 K-mean block sums, for callers
// that cannot allocate. One array per GPU, held until the process ends; host
// code reaches it only through the per-device address from static_scratch().
static __device__ __align__(256) unsigned char scratch[wf::kStaticScratchBytes];

namespace wf {
namespace {

constexpr int kTokTile = 64;                 // tokens per fp8 publish block (one quantisation block)
constexpr int kMaxFramesPerTile = kTokTile + 2;

// Time-axis (cos, sin) table of the frames one publish block (at most 64
// tokens) touches, in dynamic LDS sized per launch: frames_per_tile(HW) rows
// of 32 fp64 pairs.
extern __shared__ double2 g_ttab_dyn[];
__host__ __device__ inline int frames_per_tile(int hw) {
    const int f = (kTokTile + hw - 1) / hw + 1;
    return f < kMaxFramesPerTile ? f : kMaxFramesPerTile;
}

// floor(n / d) for 0 <= n < 2^22 (every token index: the host keeps T * N
// below 2^22) as one fp32 fma, floor((n + 1/2) r) with r = 1/d rounded to
// fp32: (n + 1/2) / d lies at least 1/(2d) from an integer, and the fma's
// result is within about 2^-23 of it relative, which stays below that margin
// for n < 2^22. Runtime integer division costs tens of instructions a token.
struct SmallDiv {
    float r;
    __device__ explicit SmallDiv(int d) : r(1.0f / (float)d) {}
    __device__ int operator()(int n) const { return (int)__builtin_fmaf((float)n, r, 0.5f * r); }
};
__device__ __forceinline__ int mul24(int a, int b) { return (int)__umul24((uint32_t)a, (uint32_t)b); }
// Frame, row and column of token n of a chunk (frames of h x w patches, row-major).
struct TokenGrid {
    SmallDiv dhw, dw;
    int hw, w;
    __device__ TokenGrid(int h, int w_) : dhw(h * w_), dw(w_), hw(h * w_), w(w_) {}
    __device__ void pos(int n, int& f, int& y, int& x) const {
        f = dhw(n);
        const int r = n - mul24(f, hw);
        y = dw(r);
        x = r - mul24(y, w);
    }
};

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

// Rotate the 4 channel pairs of one 8-channel vector starting at channel c0
// (rope_cs looks up their (cos, sin), rot8 rotates), in fp64 from fp64
// (cos, sin) tables: the published page holds the rotated value rounded once
// to the page format, so the rotation itself must be accurate far below a
// bf16 (or e4m3) rounding step. In fp32 about one element in 10^5 landed on
// the other side of a bf16 rounding midpoint, which on a x20 outlier channel
// moves a score by several units.
__device__ __forceinline__ void rope_cs(double2* cs, int c0, const double2* ttab_f, const double2* hrow,
                                        const double2* wrow, int dt, int dh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = c0 + 2 * i;
        if (c < dt) cs[i] = ttab_f[c >> 1];
        else if (c < dt + dh) cs[i] = hrow[(c - dt) >> 1];
        else cs[i] = wrow[(c - dt - dh) >> 1];
    }
}
__device__ __forceinline__ void rot8(const float* x, double* y, const double2* cs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = x[2 * i], b = x[2 * i + 1];
        y[2 * i] = fma(a, cs[i].x, -(b * cs[i].y));
        y[2 * i + 1] = fma(a, cs[i].y, b * cs[i].x);
    }
}
__device__ __forceinline__ void rope8(const float* x, double* y, int c0, const double2* ttab_f,
                                      const double2* hrow, const double2* wrow, int dt, int dh) {
    double2 cs[4];
    rope_cs(cs, c0, ttab_f, hrow, wrow, dt, dh);
    rot8(x, y, cs);
}

// Rounding an fp64 value once into bf16 (or e4m3) through fp32: the fp32
// nearest value y can only mislead the narrow format's nearest-even rounding
// when y lands exactly on one of that format's rounding midpoints while x does
// not (double rounding). Such y (bf16: low 16 bits 0x8000) are rare, about
// one value in 2^16; only they are moved one fp32 step toward x, off the
// midpoint, so the narrow rounding goes to x's side. An exact tie stays on the
// midpoint and is rounded to even, as the fp64 value would be.
__device__ __forceinline__ float off_midpoint(float y, double x) {
    const double yd = (double)y;
    const uint32_t b = __float_as_uint(y);          // sign-magnitude: +1 moves away from zero
    return fabs(yd) < fabs(x) ? __uint_as_float(b + 1u) : (fabs(yd) > fabs(x) ? __uint_as_float(b - 1u) : y);
}

__device__ __forceinline__ uint4 pack8_f64(const double* y) {
    float f[8];
    bool mid = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        f[e] = (float)y[e];
        mid |= (__float_as_uint(f[e]) & 0xFFFFu) == 0x8000u;
    }
    if (mid) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((__float_as_uint(f[e]) & 0xFFFFu) == 0x8000u) f[e] = off_midpoint(f[e], y[e]);
    }
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

// fp64 time-axis (cos, sin) of the frames f_lo .. f_lo + nf - 1 of published
// slot sr (the slot's absolute time offset plus the frame).
template <typename Args>
__device__ __forceinline__ void fill_ttab(double2 (*ttab)[32], const Args& a, int sr, int f_lo, int nf) {
    const int hp = a.dt >> 1;
    for (int i = threadIdx.x; i < nf * hp; i += blockDim.x) {
        const int fi = i / hp, m = i - fi * hp;
        const double phi = (double)(slot_t0(a, sr) + f_lo + fi) * a.omega_t[m];
        double sn, cs;
        sincos(phi, &sn, &cs);
        ttab[fi][m] = make_double2(cs, sn);
    }
}

// grid: (ceil(N / TOK), heads / HPB, nslots); block 256. One block rotates
// and publishes TOK = 256 / (D/8) tokens (16 at D = 128) of HPB heads of one
// slot. A thread owns one token and one 8-channel group in each of the HPB
// heads: the rotation's (cos, sin) depend on the token and channel only, so
// one lookup serves HPB heads of Q and of K, and a token's input reads are
// HPB * 2*D contiguous bytes of its row. Reads run along channels (coalesced
// rows of the projection output); page writes run along tokens, so K and V
// are transposed through LDS.
template <int D, bool IN_FP32, int HPB>
__global__ __launch_bounds__(256) void publish_bf16_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    constexpr int TOK = 256 / CPR;                   // tokens per block
    double2 (*ttab)[32] = reinterpret_cast<double2 (*)[32]>(g_ttab_dyn);   // time-axis (cos, sin), this tile's frames
    __shared__ __align__(16) uint4 kst[HPB * CPR * TOK];     // K vectors, [head][ch][tok ^ (ch & 7)]
    __shared__ __align__(16) uint16_t vst[HPB * TOK * D];    // V rows, [head][tok][d]

    const int tid = threadIdx.x;
    const int sr = blockIdx.z;
    const int s = a.slot_first + sr;
    const int h0 = blockIdx.y * HPB;
    const int n0 = blockIdx.x * TOK;
    const int p = a.T - 1 - s;                       // context position of slot s
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int n_hi = min(n0 + TOK, a.N) - 1;
    const int nf = n_hi / HW - f_lo + 1;
    const int tk = tid / CPR, ch = tid - tk * CPR;
    const int n = n0 + tk;
    const bool live = n < a.N;

    // the time-axis table is built first (by the block's first threads only),
    // then every row load of this thread is issued: the fp64 sincos and the
    // held rows do not need registers at the same time (rows past the chunk
    // are clamped to its last row and not used)
    fill_ttab(ttab, a, sr, f_lo, nf);
    const int64_t e0 = ((int64_t)sr * a.N + min(n, a.N - 1)) * a.row_stride + (int64_t)h0 * D + ch * 8;
    Raw8<IN_FP32> kin[HPB], qin[HPB], vin[HPB];
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
        kin[hh].load(a.k, e0 + hh * D);
        vin[hh].load(a.v, e0 + hh * D);
        if (a.q) qin[hh].load(a.q, e0 + hh * D);
    }
    __syncthreads();

    if (live) {
        // V first: its rows leave the registers before the rotation needs them
#pragma unroll
        for (int hh = 0; hh < HPB; ++hh) {
            float x[8];
            vin[hh].unpack(x);
            *reinterpret_cast<uint4*>(&vst[(hh * TOK + tk) * D + ch * 8]) = pack8(x);
        }
        const TokenGrid grid(a.frame_h, a.frame_w);
        int f, yy, xw;
        grid.pos(n, f, yy, xw);
        double2 cs[4];                               // one lookup for every head and for Q and K
        rope_cs(cs, ch * 8, ttab[f - f_lo], a.htab + yy * (a.dh >> 1), a.wtab + xw * (a.dw >> 1), a.dt, a.dh);
#pragma unroll
        for (int hh = 0; hh < HPB; ++hh) {
            float x[8];
            double r[8];
            kin[hh].unpack(x);
            rot8(x, r, cs);
            kst[(hh * CPR + ch) * TOK + (tk ^ (ch & 7))] = pack8_f64(r);
            if (a.q) {
                qin[hh].unpack(x);
                rot8(x, r, cs);
                uint16_t* qp = static_cast<uint16_t*>(a.q_out) +
                               (((int64_t)s * a.heads + h0 + hh) * a.N + n) * D + ch * 8;
                st16(qp, pack8_f64(r));
            }
        }
    }
    __syncthreads();

    const SmallDiv dpt(a.pt);
    // K pages: one 16-byte vector (8 channels of one token) per thread, tokens fastest
    for (int j = tid; j < HPB * CPR * TOK; j += 256) {
        const int hc = j / TOK, t = j - hc * TOK;    // hc = head * CPR + channel vector
        const int hh = hc / CPR, c = hc - hh * CPR;
        const int nn = n0 + t;
        if (nn >= a.N) continue;
        const int pg = dpt(nn), tok = nn - mul24(pg, a.pt);
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + h0 + hh) * a.pt * D;
        st16(static_cast<uint16_t*>(a.kpage) + k_elem(base, a.pt, tok, c * 8), kst[hc * TOK + (t ^ (c & 7))]);
    }
    // V pages: one vector of 8 consecutive tokens of one channel per thread,
    // channels fastest. N and pages are multiples of 8, so a group never
    // straddles a page.
    for (int j = tid; j < HPB * (TOK / 8) * D; j += 256) {
        const int hk = j / D, d = j - hk * D;        // hk = head * (TOK / 8) + token group
        const int hh = hk / (TOK / 8), kc = hk - hh * (TOK / 8);
        const int nn = n0 + kc * 8;
        if (nn >= a.N) continue;
        const uint16_t* vrow = vst + (hh * TOK + kc * 8) * D + d;
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (uint32_t)vrow[(2 * r) * D] | ((uint32_t)vrow[(2 * r + 1) * D] << 16);
        const int pg = dpt(nn), tok = nn - mul24(pg, a.pt);
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + h0 + hh) * a.pt * D;
        st16(a.vpage + v_elem(base, D, tok, d), make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 publish. Q and K are quantised per 64-token block of their chunk
// (blocks restart at each chunk start, so a publish block is exactly one
// quantisation block): scale = fp32 absmax / 448 (IEEE divide, 1 for an
// all-zero block), code = round-to-nearest-even of value / scale, saturating
// at +-448, every decision taken on the fp64 value. K first has its chunk's
// per-channel mean removed, the mean rounded to fp32; attention adds it back
// exactly as q . mean. V stays bf16.
//
// Three launches with fixed summation orders: kmean_partial_kernel writes the
// fp64 column sums of each 64-token block of RoPE'd K into scratch
// (kpart[published slot][head][block][D]), kmean_reduce_kernel adds a chunk's
// block sums in block order into its fp32 mean, and publish_fp8_kernel
// quantises and publishes Q, K and V.

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

// An fp32 value on an e4m3 rounding midpoint, or in e4m3's subnormal range
// (below 2^-6), where the midpoints are the odd multiples of 2^-10: the two
// cases in which rounding x to fp32 first could change its e4m3 rounding.
__device__ __forceinline__ bool e4m3_suspect(float y) {
    const uint32_t b = __float_as_uint(y);
    return (b & 0xFFFFFu) == 0x80000u || fabsf(y) < 0.015625f;
}

// x / scale to nearest even e4m3 for 8 values: the quotient in fp64 from the
// reciprocal r = 1/scale (correctly rounded) and one remainder correction
// (q0 = x r, e = x - q0 scale exactly by fma, q = q0 + e r), rounded to fp32;
// a value that lands on an e4m3 midpoint or in the subnormal range is moved
// off the midpoint toward the fp64 quotient (see off_midpoint), the exact
// e4m3 rounding of a subnormal-range value being taken on fp32 values within
// one step of 2^-30 of it.
__device__ __forceinline__ uint2 quant8(const double* x, double sc, double r) {
    float q[8];
    double qd[8];
    bool sus = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double q0 = x[e] * r;
        const double rem = fma(-q0, sc, x[e]);
        qd[e] = fma(rem, r, q0);
        q[e] = (float)qd[e];
        sus |= e4m3_suspect(q[e]);
    }
    if (sus) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!e4m3_suspect(q[e])) continue;
            if (fabsf(q[e]) < 0.015625f) {
                // subnormal range: the nearest-even multiple of 2^-9, computed
                // exactly in fp64 (the value is far inside fp64's range)
                const double m = rint(qd[e] * 512.0);
                q[e] = (float)(m * (1.0 / 512.0));
            } else {
                q[e] = off_midpoint(q[e], qd[e]);
            }
        }
    }
    return make_uint2(fp8x4(q[0], q[1], q[2], q[3]), fp8x4(q[4], q[5], q[6], q[7]));
}

// Largest |x| of the block, as fp32 (rounding is monotonic, so the fp32
// rounding of the fp64 maximum); `red` holds one float per wave.
__device__ __forceinline__ float block_absmax(float v, float* red) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

// grid (ceil(N/64), heads, nslots), 256 threads: the fp64 column sums of one
// 64-token block of RoPE'd K -> kpart[published slot][head][block][D].
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void kmean_partial_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    constexpr int ROWS = 256 / CPR;                  // token rows a pass of the block covers
    constexpr int IT = kTokTile / ROWS;
    double2 (*ttab)[32] = reinterpret_cast<double2 (*)[32]>(g_ttab_dyn);
    __shared__ double part[ROWS][D];
    const int tid = threadIdx.x;
    const int sr = blockIdx.z, head = blockIdx.y, blk = blockIdx.x;
    const int n0 = blk * kTokTile;
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int nf = (min(n0 + kTokTile, a.N) - 1) / HW - f_lo + 1;
    const int ch = tid % CPR, row = tid / CPR;
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
    const TokenGrid grid(a.frame_h, a.frame_w);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int n = n0 + row + ROWS * i;
        if (n >= a.N) break;
        int f, y, xw;
        grid.pos(n, f, y, xw);
        float x[8];
        double r[8];
        kin[i].unpack(x);
        rope8(x, r, ch * 8, ttab[f - f_lo], a.htab + y * (a.dh >> 1), a.wtab + xw * (a.dw >> 1), a.dt, a.dh);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += r[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[row][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
        for (int r = 0; r < ROWS; ++r) t += part[r][tid];
        a.kpart[(((int64_t)sr * a.heads + head) * a.nblk + blk) * D + tid] = t;
    }
}

// grid (heads, nslots), block D: kmean[group][head][d] = the chunk's block sums
// added in block order, / N, rounded to fp32.
template <int D>
__global__ void kmean_reduce_kernel(PublishArgs a) {
    const int sr = blockIdx.y, s = a.slot_first + sr, head = blockIdx.x, d = threadIdx.x;
    const int g = a.table[(a.T - 1 - s) * a.ppc] / a.ppc;
    const double* src = a.kpart + ((int64_t)sr * a.heads + head) * a.nblk * D + d;
    // eight loads in flight per iteration, summed in block order
    double sum = 0.0;
    int b = 0;
    for (; b + 8 <= a.nblk; b += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(b + u) * D];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; b < a.nblk; ++b) sum += src[(int64_t)b * D];
    a.kmean[((int64_t)g * a.heads + head) * D + d] = (float)(sum / (double)a.N);
}

// grid (ceil(N/64), heads, nslots), 256 threads: quantise and publish one
// 64-token block.
template <int D, bool IN_FP32>
__global__ __launch_bounds__(256) void publish_fp8_kernel(PublishArgs a) {
    constexpr int CPR = D / 8;                       // 8-channel vectors per token row
    constexpr int ITEMS = kTokTile * CPR / 256;      // vectors per thread
    constexpr int ROWS = 256 / CPR;                  // token rows a pass of the block covers
    constexpr int C16 = D / 16;                      // 16-byte code vectors per token row
    double2 (*ttab)[32] = reinterpret_cast<double2 (*)[32]>(g_ttab_dyn);
    __shared__ float mu[D];
    __shared__ float red[4];
    __shared__ __align__(16) uint8_t kcodes[kTokTile * D];   // [tok][16-byte vector ^ (tok % C16)]
    __shared__ __align__(16) uint16_t vst[kTokTile * D];     // V rows, [tok][d]

    const int tid = threadIdx.x;
    const int sr = blockIdx.z, s = a.slot_first + sr, head = blockIdx.y, blk = blockIdx.x;
    const int n0 = blk * kTokTile;
    const int p = a.T - 1 - s;
    const int HW = a.frame_h * a.frame_w;
    const int f_lo = n0 / HW;
    const int nf = (min(n0 + kTokTile, a.N) - 1) / HW - f_lo + 1;
    const int64_t row0 = (int64_t)sr * a.N;
    const int64_t col = (int64_t)head * D;
    const int ch = tid % CPR, row = tid / CPR;       // every item of this thread: channels ch*8 .. +7
    // rows of this thread, loaded before the tables are built (rows past the
    // chunk are clamped to its last row and not used)
    Raw8<IN_FP32> kin[ITEMS], qin[ITEMS], vin[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int tk = row + ROWS * i;
        const int64_t e0 = (row0 + min(n0 + tk, a.N - 1)) * a.row_stride + col + ch * 8;
        kin[i].load(a.k, e0);
        vin[i].load(a.v, e0);
        if (a.q) qin[i].load(a.q, e0);
    }
    fill_ttab(ttab, a, sr, f_lo, nf);
    const int g = a.table[p * a.ppc] / a.ppc;
    if (tid < D) mu[tid] = a.kmean[((int64_t)g * a.heads + head) * D + tid];
    __syncthreads();
    const TokenGrid grid(a.frame_h, a.frame_w);
    const SmallDiv dpt(a.pt);
    auto rotate = [&](const Raw8<IN_FP32>& in, int n, double* out) {
        int f, y, xw;
        grid.pos(n, f, y, xw);
        float x[8];
        in.unpack(x);
        rope8(x, out, ch * 8, ttab[f - f_lo], a.htab + y * (a.dh >> 1), a.wtab + xw * (a.dw >> 1), a.dt, a.dh);
    };

    // V staged for the page stores
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int tk = row + ROWS * i;
        if (n0 + tk >= a.N) continue;
        float x[8];
        vin[i].unpack(x);
        *reinterpret_cast<uint4*>(&vst[tk * D + ch * 8]) = pack8(x);
    }
    // Q: rotate, block absmax, codes, scale (no mean)
    if (a.q) {
        double qx[ITEMS][8];
        float qm = 0.f;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int n = n0 + row + ROWS * i;
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[i][e] = 0.0;
            if (n >= a.N) continue;
            rotate(qin[i], n, qx[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) qm = fmaxf(qm, (float)fabs(qx[i][e]));
        }
        qm = block_absmax(qm, red);
        const float qs = qm > 0.f ? qm / 448.f : 1.f;
        const double qr = 1.0 / (double)qs;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int n = n0 + row + ROWS * i;
            if (n >= a.N) continue;
            uint8_t* qp = static_cast<uint8_t*>(a.q_out) + (((int64_t)s * a.heads + head) * a.N + n) * D + ch * 8;
            *reinterpret_cast<uint2*>(qp) = quant8(qx[i], (double)qs, qr);
        }
        if (tid == 0) a.q_scales[((int64_t)s * a.heads + head) * a.nblk + blk] = qs;
    }
    // K: rotate, subtract the mean, block absmax, codes, per-token scales
    double kx[ITEMS][8];
    float km = 0.f;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int n = n0 + row + ROWS * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[i][e] = 0.0;
        if (n >= a.N) continue;
        rotate(kin[i], n, kx[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kx[i][e] -= (double)mu[ch * 8 + e];
            km = fmaxf(km, (float)fabs(kx[i][e]));
        }
    }
    km = block_absmax(km, red);
    const float ks = km > 0.f ? km / 448.f : 1.f;
    const double kr = 1.0 / (double)ks;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int tk = row + ROWS * i;
        if (n0 + tk >= a.N) continue;
        const int v16 = ch >> 1;                     // 16-byte vector of this 8-channel group
        *reinterpret_cast<uint2*>(&kcodes[(tk * C16 + (v16 ^ (tk % C16))) * 16 + (ch & 1) * 8]) =
            quant8(kx[i], (double)ks, kr);
    }
    __syncthreads();
    // K code pages: one 16-byte vector (16 channels of one token) per thread, tokens fastest
    for (int j = tid; j < C16 * kTokTile; j += 256) {
        const int v16 = j / kTokTile, tk = j - v16 * kTokTile;
        const int n = n0 + tk;
        if (n >= a.N) continue;
        const int pg = dpt(n), tok = n - mul24(pg, a.pt);
        const int phys = a.table[p * a.ppc + pg];
        const int64_t base = ((int64_t)phys * a.heads + head) * a.pt * D;
        st16(static_cast<uint8_t*>(a.kpage) + k8_byte(base, a.pt, tok, v16 * 16),
             *reinterpret_cast<const uint4*>(&kcodes[(tk * C16 + (v16 ^ (tk % C16))) * 16]));
    }
    if (tid < kTokTile && n0 + tid < a.N) {
        const int n = n0 + tid;
        const int pg = dpt(n), tok = n - mul24(pg, a.pt);
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
        const int pg = dpt(n), tok = n - mul24(pg, a.pt);
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
    const size_t tbytes = (size_t)frames_per_tile(a.frame_h * a.frame_w) * 32 * sizeof(double2);
    if (!fp8) {
        // heads per block: 4 where they divide the head count (one (cos, sin)
        // lookup per token and channel serves 4 heads; measured 2% faster
        // than one head in 32-token blocks at the Wan shapes, 2 heads equal,
        // 1 head in 16-token blocks 10% slower), else 2 or 1; fp32 inputs (a
        // full-precision check mode) take one, as their rows take twice the
        // registers
        constexpr int TOK = 256 / (D / 8);
        const int hpb = IN_FP32 ? 1 : a.heads % 4 == 0 ? 4 : a.heads % 2 == 0 ? 2 : 1;
        const dim3 gb((a.N + TOK - 1) / TOK, a.heads / hpb, a.nslots);
        if (hpb == 4) hipLaunchKernelGGL((publish_bf16_kernel<D, IN_FP32, (IN_FP32 ? 1 : 4)>), gb, dim3(256), tbytes, st, a);
        else if (hpb == 2) hipLaunchKernelGGL((publish_bf16_kernel<D, IN_FP32, (IN_FP32 ? 1 : 2)>), gb, dim3(256), tbytes, st, a);
        else hipLaunchKernelGGL((publish_bf16_kernel<D, IN_FP32, 1>), gb, dim3(256), tbytes, st, a);
        return hipGetLastError();
    }
    const dim3 grid((a.N + kTokTile - 1) / kTokTile, a.heads, a.nslots);
    hipLaunchKernelGGL((kmean_partial_kernel<D, IN_FP32>), grid, dim3(256), tbytes, st, a);
    hipLaunchKernelGGL((kmean_reduce_kernel<D>), dim3(a.heads, a.nslots), dim3(D), 0, st, a);
    hipLaunchKernelGGL((publish_fp8_kernel<D, IN_FP32>), grid, dim3(256), tbytes, st, a);
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this GPU's copy of `scratch` (the array's name is a host
// stand-in, not a device address), looked up once per device with that device
// current.
hipError_t static_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_publish(const PublishArgs& a, bool fp8, hipStream_t st) {
    if (a.D == 128) return a.in_fp32 ? launch_publish_t<128, true>(a, fp8, st) : launch_publish_t<128, false>(a, fp8, st);
    if (a.D == 64) return a.in_fp32 ? launch_publish_t<64, true>(a, fp8, st) : launch_publish_t<64, false>(a, fp8, st);
    return hipErrorInvalidValue;
}


}  // namespace wf
