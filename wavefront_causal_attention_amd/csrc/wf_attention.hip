// Wavefront attention over the paged K/V context, bf16 MFMA, gfx950.
//
// One launch covers every (query slot, head, query tile) of the round. Query
// slot s reads the context prefix [0, (T-s)*N) - anchor, clean history, store
// and the live slots that are not noisier than s - which is exactly the mask
// M_WF(s, j) = 1[j >= s] with full attention inside each chunk (Wave Forcing,
// hyper.ai summary, section "Method"; e-cogni.com.br, "Como funciona"). The
// key loop simply stops at the prefix end, so masked slot pairs are skipped as
// whole tiles and their pages are never read.
//
// Per workgroup: 128 query rows of one (slot, head), 4 waves of 32 rows.
// Per 64-key tile, each wave computes
//   S^T[key][query] = K Q^T      (v_mfma_f32_32x32x16_bf16, K from LDS, Q in VGPRs)
//   O^T[d][query]  += V^T P^T    (V^T from LDS, P^T from the S^T accumulators)
// so a lane owns one query row throughout: the softmax max and sum are in-lane
// except one exchange between the two 32-lane halves.
#include <hip/hip_runtime.h>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;         // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int kRescaleLog2 = 8; // running max may lag the true max by up to 2^8

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Position of a flat context key index, tracked incrementally tile by tile.
struct KeyCursor {
    int g;      // flat key index
    int p;      // context position (chunk)
    int pg;     // page within the chunk
    int tok;    // token within the page
    __device__ void init(int g0, int N, int pt) {
        g = g0;
        p = g0 / N;
        const int r = g0 - p * N;
        pg = r / pt;
        tok = r - pg * pt;
    }
    __device__ void step(int n, int pt, int ppc) {
        g += n;
        tok += n;
        while (tok >= pt) {
            tok -= pt;
            if (++pg == ppc) { pg = 0; ++p; }
        }
    }
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KST = D + 8;     // K tile row stride in LDS (elements), 16B pad
    constexpr int VST = BN + 8;    // V^T tile row stride in LDS
    constexpr int KSTEPS = D / 16; // MFMA k-steps of QK^T
    constexpr int DB = D / 32;     // 32-wide d blocks of the output
    constexpr int CPR = D / 8;     // 16-byte vectors per K row
    constexpr int KRT = D / 32;    // consecutive K rows a thread loads per tile
    constexpr int VCT = D / 32;    // V^T vectors a thread loads per tile

    __shared__ __align__(16) uint16_t klds[2][BN * KST];
    __shared__ __align__(16) uint16_t vlds[2][D * VST];
    __shared__ int ptab[kMaxTablePages];

    const int tid = threadIdx.x;
    int w = blockIdx.x;
    const int per_slot = a.heads * a.qtiles;
    const int sr = w / per_slot;
    w -= sr * per_slot;
    const int head = w / a.qtiles;
    const int qt = w - head * a.qtiles;
    const int s = a.slot_first + sr;
    const int N = a.N, pt = a.pt, ppc = a.ppc;
    const int nkeys = (a.T - s) * N;               // legal prefix of slot s
    const int ntiles = (nkeys + BN - 1) / BN;

    for (int i = tid; i < a.T * ppc; i += 256) ptab[i] = a.table[i];

    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int qrow = qt * BM + wave * 32 + l32;

    // Q^T operand fragments: lane holds Q[qrow][16*ks + 8*hf .. +7]
    bf16x8 qf[KSTEPS];
    {
        const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                             (((int64_t)s * a.heads + head) * N + min(qrow, N - 1)) * D + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 u = *reinterpret_cast<const uint4*>(qb + 16 * ks);
            if (qrow >= N) u = make_uint4(0, 0, 0, 0);
            qf[ks] = as_bf16x8(u);
        }
    }

    const uint16_t* kpage = static_cast<const uint16_t*>(a.kpage);
    const uint16_t* vpage = a.vpage;
    const int64_t head_stride_k = (int64_t)pt * D;     // one (page, head) block of K
    const int kr0 = KRT * (tid / CPR);                   // first K row of this thread
    const int kdc = tid % CPR;
    const int vkc = tid & 7;                             // 8-key group of this thread
    const int vdd = tid >> 3;                            // first V^T row of this thread
    KeyCursor kc, vc;
    kc.init(kr0, N, pt);
    vc.init(8 * vkc, N, pt);

    uint4 kreg[KRT], vreg[VCT];
    auto load_tile = [&]() {
        if (kc.g < nkeys) {
            const int phys = ptab[kc.p * ppc + kc.pg];
            const uint16_t* src = kpage + ((int64_t)phys * a.heads + head) * head_stride_k +
                                  (int64_t)kc.tok * D + kdc * 8;
#pragma unroll
            for (int i = 0; i < KRT; ++i) kreg[i] = *reinterpret_cast<const uint4*>(src + i * D);
        } else {
#pragma unroll
            for (int i = 0; i < KRT; ++i) kreg[i] = make_uint4(0, 0, 0, 0);
        }
        if (vc.g < nkeys) {
            const int phys = ptab[vc.p * ppc + vc.pg];
            const uint16_t* src = vpage + ((int64_t)phys * a.heads + head) * (int64_t)D * pt + vc.tok;
#pragma unroll
            for (int i = 0; i < VCT; ++i)
                vreg[i] = *reinterpret_cast<const uint4*>(src + (int64_t)(vdd + 32 * i) * pt);
        } else {
#pragma unroll
            for (int i = 0; i < VCT; ++i) vreg[i] = make_uint4(0, 0, 0, 0);
        }
        kc.step(BN, pt, ppc);
        vc.step(BN, pt, ppc);
    };
    // V^T rows are stored with keys permuted inside each 16-key group so that
    // lane half hf reads its 8 keys {4hf..4hf+3, 8+4hf..8+4hf+3} as one vector:
    // position 8h+i holds key 4h+i, position 8h+4+i holds key 8+4h+i.
    auto store_tile = [&](int buf) {
        uint16_t* kl = klds[buf];
#pragma unroll
        for (int i = 0; i < KRT; ++i)
            *reinterpret_cast<uint4*>(kl + (kr0 + i) * KST + kdc * 8) = kreg[i];
        uint16_t* vl = vlds[buf];
        const int g16 = vkc >> 1, half = vkc & 1;
#pragma unroll
        for (int i = 0; i < VCT; ++i) {
            uint16_t* row = vl + (vdd + 32 * i) * VST + 16 * g16;
            *reinterpret_cast<uint2*>(row + 4 * half) = make_uint2(vreg[i].x, vreg[i].y);
            *reinterpret_cast<uint2*>(row + 8 + 4 * half) = make_uint2(vreg[i].z, vreg[i].w);
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    float m_run = -INFINITY;   // running max of raw scores (may lag by < 2^8 in exp2 units)
    float l_run = 0.f;         // this lane's partial row sum
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    const float c = a.scale_log2;

    __syncthreads();           // ptab visible
    load_tile();
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const bool more = t + 1 < ntiles;
        if (more) load_tile();

        // S^T = K Q^T for two 32-key blocks
        f32x16 sacc[2];
        const uint16_t* kl = klds[buf];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
            const uint16_t* krow = kl + (32 * kb + l32) * KST + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8 ka = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * ks));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sacc[kb], 0, 0, 0);
            }
        }
        // keys past the legal prefix (last tile only)
        const int kbase = t * BN;
        if (kbase + BN > nkeys) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kb + 8 * (j >> 2) + 4 * hf + (j & 3);
                    if (kbase + key >= nkeys) sacc[kb][j] = -INFINITY;
                }
        }
        // online softmax, one query row per lane (pair of lanes l, l+32)
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__any((m_new - m_run) * c > (float)kRescaleLog2)) {
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
        // P is rounded to bf16 for the PV product; the row sum adds the same
        // rounded values (v_dot2 with (1, 1)), so the weights actually applied
        // to V are normalised exactly.
        const float mb = m_run * c;
        uint32_t pk[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j], c, -mb));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j + 1], c, -mb));
                pk[kb][j >> 1] = pack_bf16x2(p0, p1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kb][j >> 1]),
                                                        kOnes, l_run, false);
            }
        // O^T += V^T P^T over four 16-key groups
        const uint16_t* vl = vlds[buf];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t* src = pk[g >> 1] + 4 * (g & 1);
            const bf16x8 pb = as_bf16x8(make_uint4(src[0], src[1], src[2], src[3]));
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 va = as_bf16x8(
                    *reinterpret_cast<const uint4*>(vl + (32 * db + l32) * VST + 16 * g + 8 * hf));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
            }
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // normalise and store: lane holds O[qrow][32*db + 8*(j/4) + 4*hf + j%4]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
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
    if (fp8) return hipErrorNotSupported;
    AttnArgs a = a0;
    a.qtiles = (a.N + BM - 1) / BM;
    const int64_t blocks = (int64_t)a.nslots * a.heads * a.qtiles;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.D == 128)
        hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else if (a.D == 64)
        hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wf
