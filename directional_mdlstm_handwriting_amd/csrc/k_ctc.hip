// k_ctc.hip — the model head after the last MDLSTM level: height collapse, the fully-connected layer shared
// across directions, and the CTC loss with its gradient.
//
// "No Padding Please" §II / Figure 1: the network ends in one fully-connected layer shared by the four scan
// directions (here applied to their sum, the layer output; the bias counted once), and is trained with CTC
// (the pages' reference [13], Graves et al. 2006). The image height is collapsed by summing the rows, so
// example e gives T = w_e frames Y[t] = sum_r y_e[r][t]; logits z[t] = Y[t] Wfc + b over K classes (class 0
// is the blank), log-probabilities by a softmax over each frame, and the loss -ln p(l | x) by the CTC
// forward-backward recursion over the blank-padded label l' = (0, l1, 0, ..., lU, 0) in log space: alpha
// over prefixes, beta over suffixes, both including the frame's own probability. The gradient of the loss
// with respect to the logits is dz_t(k) = y_t(k) - exp(lse_{s: l'_s = k}(alpha_t(s) + beta_t(s)) - ln p -
// ln y_t(k)); dY = dz Wfc^T reaches every row of the frame (the collapse was a sum).
//
// One workgroup per example runs the whole head: the frames are few and short, and a single launch keeps
// the head at one dispatch plus a fixed-order reduction of the per-example weight-gradient partials. The
// example's intermediate arrays and a copy of Wfc sit in LDS when they fit (the loops over hidden units,
// classes and frames then read LDS), else in the caller's workspace, where a slot per example holds every
// size the layout allows. alpha and beta advance together, half the workgroup each, one barrier per frame.
#include "kernels.h"
#include "devmath.h"

#include <cmath>

namespace mdl {

namespace {

constexpr int CTC_THREADS = 1024;
constexpr float kLn2 = 0.693147180559945309f;

__device__ inline float flog(float x) { return __builtin_amdgcn_logf(x) * kLn2; }  // v_log_f32 is log2

// ln(e^a + e^b) for float64 a, b; -inf when both are. The correction ln(1 + e^-|a-b|) lies in [0, ln 2], so
// float32 hardware exp2 / log2 give it to about 1e-7 absolute, which is all the sum needs.
__device__ inline double lse2(double a, double b) {
    const double m = fmax(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + (double)flog(1.0f + fexp((float)-fabs(a - b)));
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}


// Example e = blockIdx.x. Its arrays: Y [Tmax][H], log-probabilities [Tmax][K], dz [Tmax][K] (float),
// then, 8-byte aligned, log alpha and log beta [Tmax][Smax] (double). SH: they sit in LDS, after a copy of
// Wfc [H][K] and before the blank-padded label l' (Smax ints); otherwise in the example's workspace slot,
// and Wfc and the labels are read from global memory. alpha and beta are kept in float64: in log space
// they grow like the loss (hundreds for long lines), where a float32 unit in the last place would already
// move the gradient's posterior by about 1e-4; the per-frame log-probabilities stay float32. The weight-gradient partial [(H + 1)][K] (row H: the bias) goes to part + e (H + 1) K
// of the workspace. An example whose label offsets fall outside [0, nlab] or decrease, whose label is
// longer than Umax, or holds a class outside 1..K-1, gets loss NaN and zero gradients.
template <bool SH, int KV>
__global__ __launch_bounds__(CTC_THREADS) void k_ctc_head(Dev D, const float* __restrict__ y_flat, int H,
                                                          const float* __restrict__ Wfc,
                                                          const float* __restrict__ bfc, int K,
                                                          const int32_t* __restrict__ labels,
                                                          const int32_t* __restrict__ loff, int64_t nlab, int Umax,
                                                          int Tmax, float* __restrict__ ws, float* __restrict__ loss,
                                                          float* __restrict__ dy_flat) {
    const int e = blockIdx.x;
    const int rh = D.real[4 * e + 2], T = D.real[4 * e + 3];
    const int64_t yb = D.flat_off[e] * H;
    const CtcWs W = ctc_ws(D.n, Tmax, H, K, Umax);
    const int64_t Smax = W.smax;
    extern __shared__ __align__(16) float sm[];
    // the copy of Wfc leads the LDS form; every array starts on 16 bytes
    const CtcOff O = ctc_offsets(SH ? (int64_t)H * K : 0, Tmax, H, K, Smax);
    float* const base = SH ? sm : ws + (int64_t)e * W.slot;
    const float* Wm = SH ? sm : Wfc;
    float* Y = base + O.y;
    float* LY = base + O.ly;
    float* DZ = base + O.dz;
    double* LA = reinterpret_cast<double*>(base + O.la);
    double* LB = reinterpret_cast<double*>(base + O.lb);
    int* LP = reinterpret_cast<int*>(base + O.lp);  // SH only
    float* PW = ws + W.part + (int64_t)e * (H + 1) * K;
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (SH) {
#pragma unroll 8
        for (int i = tid; i < H * K; i += nthr) sm[i] = Wfc[i];
    }

    const int64_t u0 = loff[e], u1 = loff[e + 1];
    bool bad = !(u0 >= 0 && u0 <= u1 && u1 <= nlab && u1 - u0 <= Umax);
    const int U = bad ? 0 : (int)(u1 - u0);
    for (int i = tid; i < U; i += nthr) {
        const int c = labels[u0 + i];
        bad |= c < 1 || c >= K;
    }
    if (SH)
        for (int s = tid; s < 2 * U + 1; s += nthr) LP[s] = (s & 1) ? labels[u0 + (s >> 1)] : 0;
    bad = __syncthreads_or(bad);

    // height collapse
    for (int i = tid; i < T * H; i += nthr) {
        const int t = i / H, j = i - t * H;
        const float* yp = y_flat + yb + (int64_t)t * H + j;
        const int64_t rs = (int64_t)T * H;
        float s = 0.f;
        int r = 0;
        for (; r + 4 <= rh; r += 4) {  // four rows' loads in flight, added in row order
            const float a0 = yp[r * rs], a1 = yp[(r + 1) * rs], a2 = yp[(r + 2) * rs], a3 = yp[(r + 3) * rs];
            s += a0;
            s += a1;
            s += a2;
            s += a3;
        }
        for (; r < rh; ++r) s += yp[r * rs];
        Y[i] = s;
    }
    __syncthreads();
    // logits (KV = 4: four classes per thread, 16-byte LDS reads of Wfc rows)
    const int KQ = K / KV;
    for (int i = tid; i < T * KQ; i += nthr) {
        const int t = i / KQ, k = (i - t * KQ) * KV;
        const float* yt = Y + (int64_t)t * H;
        if constexpr (KV == 4) {
            f32x4 z = {bfc[k], bfc[k + 1], bfc[k + 2], bfc[k + 3]};
            for (int j = 0; j < H; ++j) {
                const f32x4 w = *reinterpret_cast<const f32x4*>(Wm + (int64_t)j * K + k);
                const float y = yt[j];
                z = f32x4{__builtin_fmaf(y, w[0], z[0]), __builtin_fmaf(y, w[1], z[1]), __builtin_fmaf(y, w[2], z[2]),
                          __builtin_fmaf(y, w[3], z[3])};
            }
            *reinterpret_cast<f32x4*>(LY + (int64_t)t * K + k) = z;
        } else {
            float z = bfc[k];
            for (int j = 0; j < H; ++j) z = __builtin_fmaf(yt[j], Wm[(int64_t)j * K + k], z);
            LY[(int64_t)t * K + k] = z;
        }
    }
    __syncthreads();
    // log-softmax, one wave per frame
    {
        const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
        for (int t = wave; t < T; t += nw) {
            float* z = LY + (int64_t)t * K;
            float m = -INFINITY;
            for (int k = lane; k < K; k += 64) m = fmaxf(m, z[k]);
            m = wave_max(m);
            float s = 0.f;
            for (int k = lane; k < K; k += 64) s += fexp(z[k] - m);
            const float ls = m + flog(wave_sum(s));
            for (int k = lane; k < K; k += 64) z[k] -= ls;
        }
    }
    __syncthreads();

    // alpha (first half of the threads) and beta (second half), frame by frame
    const int S = 2 * U + 1;
    auto lab = [&](int s) { return SH ? LP[s] : ((s & 1) ? labels[u0 + (s >> 1)] : 0); };
    if (!bad) {
        const int half = nthr / 2;
        const bool fa = tid < half;
        const int ht = fa ? tid : tid - half;
        for (int step = 0; step < T; ++step) {
            if (fa) {
                const int t = step;
                for (int s = ht; s < S; s += half) {
                    const int c = lab(s);
                    double v;
                    if (t == 0) {
                        v = s < 2 ? 0.0 : -INFINITY;
                    } else {
                        const double* prev = LA + (int64_t)(t - 1) * Smax;
                        v = prev[s];
                        if (s >= 1) v = lse2(v, prev[s - 1]);
                        if (s >= 2 && c != 0 && c != lab(s - 2)) v = lse2(v, prev[s - 2]);
                    }
                    LA[(int64_t)t * Smax + s] = v + (double)LY[(int64_t)t * K + c];
                }
            } else {
                const int t = T - 1 - step;
                for (int s = ht; s < S; s += half) {
                    const int c = lab(s);
                    double v;
                    if (t == T - 1) {
                        v = s >= S - 2 ? 0.0 : -INFINITY;
                    } else {
                        const double* next = LB + (int64_t)(t + 1) * Smax;
                        v = next[s];
                        if (s + 1 < S) v = lse2(v, next[s + 1]);
                        if (s + 2 < S && c != 0 && c != lab(s + 2)) v = lse2(v, next[s + 2]);
                    }
                    LB[(int64_t)t * Smax + s] = v + (double)LY[(int64_t)t * K + c];
                }
            }
            __syncthreads();
        }
    }
    double lp = -INFINITY;
    if (!bad) {
        const double* last = LA + (int64_t)(T - 1) * Smax;
        lp = S > 1 ? lse2(last[S - 1], last[S - 2]) : last[0];
    }
    const bool live = !bad && lp > -INFINITY;
    if (tid == 0) loss[e] = bad ? NAN : (live ? (float)-lp : INFINITY);

    // gradient of the loss with respect to the logits
    for (int i = tid; i < T * K; i += nthr) {
        const int t = i / K, k = i - t * K;
        float g = 0.f;
        if (live) {
            const float ly = LY[i];
            const double* at = LA + (int64_t)t * Smax;
            const double* bt = LB + (int64_t)t * Smax;
            double acc = -INFINITY;
            if (k == 0) {
                for (int s = 0; s < S; s += 2) acc = lse2(acc, at[s] + bt[s]);
            } else {
                for (int s = 1; s < S; s += 2)
                    if (lab(s) == k) acc = lse2(acc, at[s] + bt[s]);
            }
            g = fexp(ly) - (float)exp(acc - lp - (double)ly);
        }
        DZ[i] = g;
    }
    __syncthreads();
    // this example's weight-gradient partial: sum over frames of Y^T dz, and of dz for the bias
    for (int i = tid; i < (H + 1) * KQ; i += nthr) {
        const int j = i / KQ, k = (i - j * KQ) * KV;
        if constexpr (KV == 4) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int t = 0; t < T; ++t) {
                const float y = j < H ? Y[(int64_t)t * H + j] : 1.f;
                const f32x4 d = *reinterpret_cast<const f32x4*>(DZ + (int64_t)t * K + k);
                acc = f32x4{__builtin_fmaf(y, d[0], acc[0]), __builtin_fmaf(y, d[1], acc[1]),
                            __builtin_fmaf(y, d[2], acc[2]), __builtin_fmaf(y, d[3], acc[3])};
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) PW[(int64_t)j * K + k + q] = acc[q];
        } else {
            float acc = 0.f;
            for (int t = 0; t < T; ++t)
                acc = __builtin_fmaf(j < H ? Y[(int64_t)t * H + j] : 1.f, DZ[(int64_t)t * K + k], acc);
            PW[(int64_t)j * K + k] = acc;
        }
    }
    // gradient of the direction sum: dY = dz Wfc^T, the same for every row of the frame
    if (dy_flat) {
        for (int i = tid; i < T * H; i += nthr) {
            const int t = i / H, j = i - t * H;
            const float* dz = DZ + (int64_t)t * K;
            const float* wr = Wm + (int64_t)j * K;
            float g = 0.f;
            if constexpr (KV == 4) {
                for (int k = 0; k < K; k += 4) {
                    const f32x4 d = *reinterpret_cast<const f32x4*>(dz + k);
                    const f32x4 w = *reinterpret_cast<const f32x4*>(wr + k);
                    g = __builtin_fmaf(d[0], w[0], g);
                    g = __builtin_fmaf(d[1], w[1], g);
                    g = __builtin_fmaf(d[2], w[2], g);
                    g = __builtin_fmaf(d[3], w[3], g);
                }
            } else {
                for (int k = 0; k < K; ++k) g = __builtin_fmaf(dz[k], wr[k], g);
            }
            for (int r = 0; r < rh; ++r) dy_flat[yb + ((int64_t)r * T + t) * H + j] = g;
        }
    }
}

// dWfc / dbfc from the per-example partials in a fixed order: RW_O outputs per workgroup, RW_G thread groups
// each summing the examples e = g, g + RW_G, ... (eight loads in flight), then the groups' sums in order g
constexpr int RW_O = 64, RW_G = 4;
__global__ __launch_bounds__(RW_O * RW_G) void k_ctc_wreduce(const float* __restrict__ part, int n, int HK1, int HK,
                                                             float* __restrict__ dW, float* __restrict__ db) {
    __shared__ float red[RW_G][RW_O];
    const int o = threadIdx.x % RW_O, g = threadIdx.x / RW_O;
    const int i = blockIdx.x * RW_O + o;
    float acc = 0.f;
    if (i < HK1) {
        int e = g;
        for (; e + 7 * RW_G < n; e += 8 * RW_G) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(e + u * RW_G) * HK1 + i];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; e < n; e += RW_G) acc += part[(int64_t)e * HK1 + i];
    }
    red[g][o] = acc;
    __syncthreads();
    if (g == 0 && i < HK1) {
        float t = red[0][o];
#pragma unroll
        for (int q = 1; q < RW_G; ++q) t += red[q][o];
        if (i < HK) dW[i] = t;
        else db[i - HK] = t;
    }
}

}  // namespace

size_t ctc_lds_bytes(int Tmax, int H, int K, int Umax) {
    const int64_t smax = 2 * (int64_t)Umax + 1;
    return 4 * (size_t)(ctc_offsets((int64_t)H * K, Tmax, H, K, smax).lp + smax);
}

hipError_t launch_ctc_head(const Dev& D, const float* y_flat, int H, const float* Wfc, const float* bfc, int K,
                           const int32_t* labels, const int32_t* label_off, int64_t nlab, int Umax, int Tmax,
                           float* ws, float* loss, float* dy_flat, float* dW, float* db, size_t lds_limit,
                           hipStream_t st) {
    const size_t lds = ctc_lds_bytes(Tmax, H, K, Umax);  // whole bytes of the in-LDS form
    // in LDS, classes in fours where K allows (aligned 16-byte rows); in the workspace, one at a time
    auto kern = lds > lds_limit ? k_ctc_head<false, 1> : (K % 4 == 0 ? k_ctc_head<true, 4> : k_ctc_head<true, 1>);
    launch(kern, dim3(D.n), dim3(CTC_THREADS), lds > lds_limit ? 0 : lds, st, D, y_flat, H, Wfc, bfc, K, labels,
           label_off, nlab, Umax, Tmax, ws, loss, dy_flat);
    if (dW) {
        const CtcWs W = ctc_ws(D.n, Tmax, H, K, Umax);
        const int HK1 = (H + 1) * K;
        launch(k_ctc_wreduce, dim3((HK1 + RW_O - 1) / RW_O), dim3(RW_O * RW_G), 0, st, ws + W.part, D.n, HK1,
               H * K, dW, db);
    }
    return hipGetLastError();
}

}  // namespace mdl
