// Recurrent decode step of the gated delta rule for gfx950: one new token per
// (sequence, head), applied to the fp32 state in place.
//
// One token of the recurrence (paper note "Gated Delta Networks: Improving Mamba2 with
// Delta Rule", mechanism paragraph; module page "Gated DeltaNet", "How It Works"):
//   S <- alpha S + beta (v - alpha S k) k^T,     o = S q   (the updated state)
// Each state row s_i (one v index) is independent:
//   a_i = s_i . k,  b_i = s_i . q,  c_i = beta (v_i - alpha a_i),
//   s_i <- alpha s_i + c_i k,        o_i = alpha b_i + c_i (k . q)
// so every row is read once and written once: the step streams the state through HBM.
//
// With a channel-wise decay (one alpha per key channel, g [N, H, d_k]; record "LIT-137",
// "Standing in the anthology") the decay scales the state's columns instead:
//   s~_i = s_i * alpha,  a_i = s~_i . k,  b_i = s~_i . q,  c_i = beta (v_i - a_i),
//   s_i <- s~_i + c_i k,  o_i = b_i + c_i (k . q).
// With decoupled erase and write gates e [N, H, d_k], w [N, H, d_v] (record "LIT-137",
// "Standing in the anthology") the erased read runs along e * k and the value is w_i v_i:
//   a_i = s~_i . (e * k),  c_i = w_i v_i - a_i.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// One DPP lane permutation within each 16-lane row (control word fixed at compile time).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row (all 16 lanes receive the total):
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    return x;
}

// One work-group per (sequence, head). Its 256 lanes form 16 groups of 16; group g owns
// rows g, g+16, ...; within a group, lane l16 owns the columns 4 l16 + 0..3 of each 64-column
// half of a row, so that every load and store of the state covers whole 256-byte runs
// (16 lanes x 16 bytes, full cache lines). The state is streamed with non-temporal loads and
// stores: each byte is touched once per step.
template <typename TS, typename TO, int DK, int DV, bool CW, bool DEC>
__global__ __launch_bounds__(256) void decode_kernel(DecodeProblem p) {
    constexpr int EPL = DK / 16;   // state columns per lane
    constexpr int NH = EPL / 4;    // 16-byte pieces per lane and row
    constexpr int HW = DK / NH;    // columns between a lane's pieces
    constexpr int RPG = DV / 16;   // rows per lane group
    const long pr = blockIdx.x;
    const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
    auto col = [&](int e) { return HW * (e >> 2) + 4 * l16 + (e & 3); };   // column of value e

    float kf[EPL], qf[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kf[e] = to_f32(static_cast<const TS*>(p.k)[pr * DK + col(e)]);
        qf[e] = to_f32(static_cast<const TS*>(p.q)[pr * DK + col(e)]);
    }
    float ke[EPL];   // the key the erased read runs along
#pragma unroll
    for (int e = 0; e < EPL; ++e) ke[e] = DEC ? p.erase[pr * DK + col(e)] * kf[e] : kf[e];
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) kq += kf[e] * qf[e];
    kq = row16_sum(kq);
    const float alpha = CW ? 1.f : __expf(p.g[pr]);
    const float beta = DEC ? 1.f : p.beta[pr];
    float af[EPL];   // channel-wise decay of this lane's columns
#pragma unroll
    for (int e = 0; e < EPL; ++e) af[e] = CW ? __expf(p.g[pr * DK + col(e)]) : 1.f;

    float* st = p.state + pr * (long)DV * DK + 4 * l16;
    const TS* vp = static_cast<const TS*>(p.v) + pr * DV;
    TO* op = static_cast<TO*>(p.o) + pr * DV;

    float s[RPG][EPL];
    float vr[RPG];
#pragma unroll
    for (int it = 0; it < RPG; ++it) {
        const int row = grp + 16 * it;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(st + (long)row * DK + HW * (e >> 2)));
            s[it][e] = x[0]; s[it][e + 1] = x[1]; s[it][e + 2] = x[2]; s[it][e + 3] = x[3];
        }
        if constexpr (CW) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s[it][e] *= af[e];
        }
        vr[it] = to_f32(vp[row]);
        if constexpr (DEC) vr[it] *= p.write[pr * DV + row];
    }
#pragma unroll
    for (int it = 0; it < RPG; ++it) {
        const int row = grp + 16 * it;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            sk += s[it][e] * ke[e];
            sq += s[it][e] * qf[e];
        }
        sk = row16_sum(sk);
        sq = row16_sum(sq);
        const float c = beta * (vr[it] - alpha * sk);
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const f32x4_t x = {alpha * s[it][e] + c * kf[e], alpha * s[it][e + 1] + c * kf[e + 1],
                               alpha * s[it][e + 2] + c * kf[e + 2], alpha * s[it][e + 3] + c * kf[e + 3]};
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(st + (long)row * DK + HW * (e >> 2)));
        }
        if (l16 == 0) op[row] = from_f32<TO>(alpha * sq + c * kq);
    }
}

template <typename TS, typename TO, int DK, int DV>
static hipError_t decode_launch(const DecodeProblem& p, hipStream_t s) {
    const dim3 grid((unsigned)((long)p.N * p.H));
    if (p.erase) return launch(decode_kernel<TS, TO, DK, DV, true, true>, grid, dim3(256), s, p);
    if (p.channel_gate) return launch(decode_kernel<TS, TO, DK, DV, true, false>, grid, dim3(256), s, p);
    return launch(decode_kernel<TS, TO, DK, DV, false, false>, grid, dim3(256), s, p);
}

template <typename TS, typename TO>
static hipError_t decode_dispatch(const DecodeProblem& p, hipStream_t s) {
    if (p.dk == 64)
        return p.dv == 64 ? decode_launch<TS, TO, 64, 64>(p, s) : decode_launch<TS, TO, 64, 128>(p, s);
    return p.dv == 64 ? decode_launch<TS, TO, 128, 64>(p, s) : decode_launch<TS, TO, 128, 128>(p, s);
}

hipError_t launch_decode(const DecodeProblem& p, hipStream_t s) {
    if ((long)p.N * p.H == 0) return hipSuccess;
    if (p.bf16)
        return p.o_bf16 ? decode_dispatch<uint16_t, uint16_t>(p, s) : decode_dispatch<uint16_t, float>(p, s);
    return p.o_bf16 ? decode_dispatch<float, uint16_t>(p, s) : decode_dispatch<float, float>(p, s);
}

}  // namespace gdn
