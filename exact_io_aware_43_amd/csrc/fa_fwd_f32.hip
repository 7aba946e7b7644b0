// Forward attention with fp32 inputs and fp32 arithmetic throughout.
//
// Same method as the 16-bit path ("FlashAttention: Faster Attention Without
// Dropping a Single Interaction", Method Deep Dive, Key designs 1 and 2): K and
// V stream through LDS in tiles, each query row keeps a running max, running
// sum and output accumulator, and only O and lse are written. Products are
// plain fp32 FMAs (no reduced-precision contraction), so the result is fp32
// attention up to reduction order.
//
// Work decomposition: a workgroup of 128 threads owns 64 query rows; the two
// threads of a lane pair split the head dimension in halves, combine their
// partial dot products with one lane exchange, and run the (identical) softmax
// bookkeeping redundantly. Each K/V tile holds 16 keys. A sliding window
// limits the visited key range and masks per key; softcapping (compiled
// instances) maps the scaled score u to cap tanh(u / cap) with the library
// tanhf before the bias.
#include "fa_device.hpp"

namespace fa {
namespace {

constexpr int F_ROWS = 64;   // query rows per workgroup
constexpr int F_NT = 128;    // threads per workgroup
constexpr int F_BC = 16;     // keys per tile

template <int D, bool CAUSAL, bool ALIBI, bool CAP>
__global__ __launch_bounds__(F_NT) void fwd_f32_kernel(Args a) {
    constexpr int DH = D / 2;
    __shared__ __attribute__((aligned(16))) float Ks[F_BC][D];
    __shared__ __attribute__((aligned(16))) float Vs[F_BC][D];

    const int tid = threadIdx.x;
    const int half = tid & 1;
    const int h = blockIdx.x, b = blockIdx.y;
    const int qt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
    int row0, len;
    seq_bounds(a, b, row0, len);
    const int q0 = qt * F_ROWS;
    if (q0 >= len) return;
    const int qi = q0 + (tid >> 1);
    const int g = h / a.G;
    const size_t ldq = (size_t)a.H * D, ldk = (size_t)a.Hkv * D;
    const float* Q = reinterpret_cast<const float*>(a.q) + (size_t)row0 * ldq + (size_t)h * D;
    const float* Kg = reinterpret_cast<const float*>(a.k) + (size_t)row0 * ldk + (size_t)g * D;
    const float* Vg = reinterpret_cast<const float*>(a.v) + (size_t)row0 * ldk + (size_t)g * D;

    float q[DH], o[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        q[c] = (qi < len) ? Q[(size_t)qi * ldq + half * DH + c] : 0.f;
        o[c] = 0.f;
    }
    const float c2 = a.scale_log2;
    const float slope2 = ALIBI ? ld_uniform(a.slopes + h) * kLog2e : 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // window bounds (causal: nothing right of the diagonal) and the keys some
    // row of the workgroup can see
    const int wl = a.wl, wr = CAUSAL ? 0 : a.wr;
    const int kend = min(len, q0 + F_ROWS + wr);
    const float cap = CAP ? a.cap_out * kLn2 : 0.f;  // cap, natural units
    for (int k0 = max(q0 - wl, 0) / F_BC * F_BC; k0 < kend; k0 += F_BC) {
        __syncthreads();
        for (int e = tid; e < F_BC * D / 4; e += F_NT) {
            const int key = e / (D / 4), c4 = e % (D / 4);
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (k0 + key < len) {
                kv = *reinterpret_cast<const float4*>(Kg + (size_t)(k0 + key) * ldk + 4 * c4);
                vv = *reinterpret_cast<const float4*>(Vg + (size_t)(k0 + key) * ldk + 4 * c4);
            }
            *reinterpret_cast<float4*>(&Ks[key][4 * c4]) = kv;
            *reinterpret_cast<float4*>(&Vs[key][4 * c4]) = vv;
        }
        __syncthreads();

        float s[F_BC];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < F_BC; ++j) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < DH; ++c) part = fmaf(q[c], Ks[j][half * DH + c], part);
            const float dot = part + __shfl_xor(part, 1);
            const int key = k0 + j;
            float t = CAP ? cap * tanhf(dot * a.cap_in) * kLog2e : dot * c2;
            if (ALIBI) {
                const float dist = (float)(qi - key);
                t -= slope2 * (CAUSAL ? dist : fabsf(dist));
            }
            if (key >= len || key > qi + wr || key < qi - wl) t = -INFINITY;
            s[j] = t;
            mt = fmaxf(mt, t);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < F_BC; ++j) {
            s[j] = exp2f(s[j] - m_use);
            ls += s[j];
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int c = 0; c < DH; ++c) {
            float acc = o[c] * alpha;
#pragma unroll
            for (int j = 0; j < F_BC; ++j) acc = fmaf(s[j], Vs[j][half * DH + c], acc);
            o[c] = acc;
        }
    }

    if (qi < len) {
        const float inv = 1.f / l_run;
        float* O = reinterpret_cast<float*>(a.out) + (size_t)row0 * ldq + (size_t)h * D + (size_t)qi * ldq;
#pragma unroll
        for (int c = 0; c < DH; ++c) O[half * DH + c] = o[c] * inv;
        if (half == 0) a.lse[((size_t)b * a.H + h) * a.N + qi] = (m_run + log2f(l_run)) * kLn2;
    }
}

template <int D, bool CAUSAL, bool ALIBI, bool CAP>
hipError_t launch(const Args& a, hipStream_t s) {
    dim3 grid(a.H, a.B, (a.N + F_ROWS - 1) / F_ROWS);
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, ALIBI, CAP>), grid, dim3(F_NT), 0, s, a);
    return hipGetLastError();
}

template <int D, bool CAP>
hipError_t launch_d(const Args& a, bool causal, bool alibi, hipStream_t s) {
    if (causal) return alibi ? launch<D, true, true, CAP>(a, s) : launch<D, true, false, CAP>(a, s);
    return alibi ? launch<D, false, true, CAP>(a, s) : launch<D, false, false, CAP>(a, s);
}

template <bool CAP>
hipError_t launch_c(const Args& a, int d, bool causal, bool alibi, hipStream_t s) {
    switch (d) {
        case 16: return launch_d<16, CAP>(a, causal, alibi, s);
        case 32: return launch_d<32, CAP>(a, causal, alibi, s);
        case 64: return launch_d<64, CAP>(a, causal, alibi, s);
        case 128: return launch_d<128, CAP>(a, causal, alibi, s);
        default: return launch_d<256, CAP>(a, causal, alibi, s);
    }
}

}  // namespace

hipError_t launch_fwd_f32(const Args& a, int d, bool causal, bool alibi, bool cap, hipStream_t s) {
    return cap ? launch_c<true>(a, d, causal, alibi, s) : launch_c<false>(a, d, causal, alibi, s);
}

}  // namespace fa
