// Beam sparse-MoE layer forward: plain CPU oracle.
//
// TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
// baseline leg may load this library. It shares no code, header or table with
// the GPU path; the two meet only through the seeded input generator.
//
// What it computes, in IEEE double, in the order the pages state it:
//   * pre-MLP RMSNorm (sandwich norm) of the hidden states, rounded once to bf16
//     [Transformers "Beam" model page, Overview: sandwich norms; FP32 numerics note;
//      BeamConfig: rms_norm_eps] -- large-chunk workload only;
//   * router logits z = x . Wr, sigmoid scores s, biased scores b = s + bias
//     [Transformers "Beam" page, Overview: sparse MoE item and FP32 routing note;
//      archdb "Beam-1.0-501B-A23B" fact sheet, MoE: gating function, load balancing];
//   * group score = sum of the two largest biased scores in the group; keep the
//     topk_group best groups; top_k experts by biased score inside them
//     [archdb fact sheet, MoE: expert groups row; Transformers "Beam" page,
//      BeamConfig: n_group, topk_group, num_experts_per_tok; news.hamidun.com
//      article, section on where Beam saves and where it pays in memory];
//   * weights = unbiased scores of the chosen experts renormalised to sum to 1,
//     times routed_scaling_factor [archdb fact sheet, MoE: renormalisation and
//     routed scaling rows; Transformers "Beam" page, BeamConfig: norm_topk_prob,
//     routed_scaling_factor];
//   * per chosen expert a SwiGLU MLP without biases, intermediate 2560
//     [Transformers "Beam" page, BeamConfig: hidden_act, moe_intermediate_size;
//      archdb fact sheet, FFN rows];
//   * y = sum of the weighted expert outputs, no shared expert [archdb fact sheet,
//     MoE: always-on experts = 0].
//   * expert-parallel share (optional): the same sum restricted to the slots whose expert
//     lies in one contiguous block of expert ids, what one GPU computes when each holds a
//     block of the experts ["Use HF Transformers" cookbook, Parallelism].
//   * after the layer (next step on the path, optional): the post-MLP half of the
//     sandwich norm on y, then the depth-scaled residual add, the k-th contribution
//     entering as r * sqrt((k-1)/k) + n / sqrt(k), where the embedding counts as the
//     first contribution and the MLP of 0-indexed layer i as contribution 2(i+1)+1
//     [Transformers "Beam" page, Overview: sandwich norms item; archdb fact sheet,
//      normalisation and residual rows; news.hamidun.com article, section on hybrid
//      attention and the unusual residual stream].
//
// Readings taken where the pages leave a step open:
//   - the bias selects only: group scores and the top-k use b, the weights use s;
//   - groups are contiguous blocks of E/n_group expert ids;
//   - ties go to the lower group / expert index;
//   - the SwiGLU output h is rounded to bf16 once before the down projection
//     (the down projection is a bf16 GEMM); y is reported without rounding;
//   - the RMSNorm output is rounded to bf16 once, x = bf16((h * r) * w).
//   - FP8 expert weights (decode, optional): the pages name FP8 checkpoints but no scaling
//     recipe, so the oracle takes the OCP Microscaling (MX) v1.0 FP8 layout: E4M3 elements
//     (OCP 8-bit floating point, bias 7, largest finite 448, no infinities) sharing one
//     power-of-two E8M0 scale per 32 consecutive k of a row, shared exponent
//     floor(log2(max |w|)) - 8, elements rounded to nearest even and saturated to +-448;
//     a block of zeros takes scale 2^0. The layer then runs on the dequantized weights.
//   - the post-MLP RMSNorm reads the unrounded y and is not rounded either: the
//     residual stream it feeds is accumulated in FP32 (archdb fact sheet, residual row).
//
// Layouts (row-major): x [T,d] bf16 bits, Wr [d,E] fp32, bias [E] fp32,
// Wg[e], Wu[e] [I,d] bf16 bits (one row per intermediate channel), Wd[e] [d,I].
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

// Round a double to the nearest bfloat16 (8 significant bits), ties to even,
// by scaling to an integer grid with exact power-of-two factors.
uint16_t bf16_round(double v) {
    if (std::isnan(v)) return 0x7fc0;
    if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
    int ex;
    std::frexp(v, &ex);                  // v = f * 2^ex, 0.5 <= |f| < 1
    int q_exp = ex - 8;                  // spacing of bf16 values around v
    if (q_exp < -133) q_exp = -133;      // subnormal spacing
    double q = std::ldexp(v, -q_exp);    // exact
    double r = std::nearbyint(q);        // round half to even (default mode)
    double out = std::ldexp(r, q_exp);   // exact when representable
    const double bf16_max = 3.38953138925153547590470800371487866880e38;
    if (std::fabs(out) > bf16_max) out = std::copysign(INFINITY, v);
    float f = (float)out;                // exact: out has <= 8 significant bits
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

template <class F>
void parallel_for(int64_t n, int nthreads, F f) {
    if (nthreads <= 1 || n <= 1) {
        for (int64_t i = 0; i < n; ++i) f(i);
        return;
    }
    if (nthreads > n) nthreads = (int)n;
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; ++t)
        th.emplace_back([=, &f]() {
            for (int64_t i = t; i < n; i += nthreads) f(i);
        });
    for (auto& x : th) x.join();
}

double sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

struct Route {
    std::vector<int32_t> idx;   // top_k expert ids, descending biased score
    std::vector<double> w;      // routing weights aligned with idx
    double gap;                 // smallest score gap at a selection boundary
};

// Routing of one token from its logits (double).
Route route_token(const double* z, const float* bias, int E, int G, int KG, int K, double S, int norm) {
    const int gsz = E / G;
    std::vector<double> s(E), b(E);
    for (int e = 0; e < E; ++e) {
        s[e] = sigmoid(z[e]);
        b[e] = s[e] + (double)bias[e];
    }
    // Group score: the two largest biased scores of the group, summed.
    std::vector<double> gs(G);
    for (int g = 0; g < G; ++g) {
        std::vector<double> v(b.begin() + (int64_t)g * gsz, b.begin() + (int64_t)(g + 1) * gsz);
        std::sort(v.begin(), v.end(), std::greater<double>());
        gs[g] = v[0] + v[1];
    }
    // Keep the KG best groups (lower index first on equal scores).
    std::vector<int> gord(G);
    std::iota(gord.begin(), gord.end(), 0);
    std::stable_sort(gord.begin(), gord.end(), [&](int a, int c) { return gs[a] > gs[c]; });
    std::vector<char> kept(G, 0);
    for (int i = 0; i < KG; ++i) kept[gord[i]] = 1;
    // Candidates: experts of kept groups; the rest are excluded outright.
    std::vector<int> cand;
    for (int e = 0; e < E; ++e)
        if (kept[e / gsz]) cand.push_back(e);
    std::stable_sort(cand.begin(), cand.end(), [&](int a, int c) { return b[a] > b[c]; });
    Route r;
    r.idx.assign(cand.begin(), cand.begin() + K);
    double sum = 0.0;
    for (int j = 0; j < K; ++j) sum += s[r.idx[j]];
    r.w.resize(K);
    for (int j = 0; j < K; ++j) r.w[j] = norm ? S * s[r.idx[j]] / sum : S * s[r.idx[j]];
    double gap = INFINITY;
    if (KG < G) gap = std::min(gap, gs[gord[KG - 1]] - gs[gord[KG]]);
    if (K < (int)cand.size()) gap = std::min(gap, b[cand[K - 1]] - b[cand[K]]);
    r.gap = gap;
    return r;
}

void logits_token(const uint16_t* xrow, const float* Wr, int d, int E, double* z) {
    for (int e = 0; e < E; ++e) z[e] = 0.0;
    for (int j = 0; j < d; ++j) {
        double xv = bf16_value(xrow[j]);
        const float* wrow = Wr + (int64_t)j * E;
        for (int e = 0; e < E; ++e) z[e] += xv * (double)wrow[e];
    }
}

// One expert applied to one token: o = Wd . bf16(silu(Wg . x) * (Wu . x)).
void expert_token(const uint16_t* xrow, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                  int d, int I, double* o) {
    std::vector<double> xv(d), h(I);
    for (int j = 0; j < d; ++j) xv[j] = bf16_value(xrow[j]);
    for (int n = 0; n < I; ++n) {
        const uint16_t* gr = wg + (int64_t)n * d;
        const uint16_t* ur = wu + (int64_t)n * d;
        double g = 0.0, u = 0.0;
        for (int j = 0; j < d; ++j) {
            g += xv[j] * bf16_value(gr[j]);
            u += xv[j] * bf16_value(ur[j]);
        }
        double a = g / (1.0 + std::exp(-g)) * u;   // silu(g) * u
        h[n] = bf16_value(bf16_round(a));
    }
    for (int c = 0; c < d; ++c) {
        const uint16_t* dr = wd + (int64_t)c * I;
        double acc = 0.0;
        for (int n = 0; n < I; ++n) acc += h[n] * bf16_value(dr[n]);
        o[c] = acc;
    }
}

}  // namespace

extern "C" {

// The bf16 rounding the oracle applies to h and to the normed x, exposed so it can be pinned.
void oracle_bf16_round(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}

// x[t,j] = bf16((h[t,j] * r_t) * w[j]), r_t = 1 / sqrt(mean_j h[t,j]^2 + eps).
void oracle_rmsnorm(const uint16_t* h, const uint16_t* w, int64_t T, int32_t d, double eps,
                    uint16_t* x_out, int32_t nthreads) {
    parallel_for(T, nthreads, [&](int64_t t) {
        const uint16_t* hr = h + t * d;
        double ss = 0.0;
        for (int j = 0; j < d; ++j) {
            double v = bf16_value(hr[j]);
            ss += v * v;
        }
        double r = 1.0 / std::sqrt(ss / d + eps);
        for (int j = 0; j < d; ++j) x_out[t * d + j] = bf16_round(bf16_value(hr[j]) * r * bf16_value(w[j]));
    });
}

// Raw router logits z [T,E] (double).
void oracle_logits(const uint16_t* x, const float* Wr, int64_t T, int32_t d, int32_t E, double* z_out,
                   int32_t nthreads) {
    parallel_for(T, nthreads, [&](int64_t t) { logits_token(x + t * d, Wr, d, E, z_out + t * E); });
}

// Routing of T tokens: idx [T,K] (descending biased score), w [T,K], gap [T]; z_out [T,E] optional.
void oracle_route(const uint16_t* x, const float* Wr, const float* bias, int64_t T, int32_t d, int32_t E,
                  int32_t G, int32_t KG, int32_t K, double S, int32_t norm, int32_t* idx_out, double* w_out,
                  double* gap_out, double* z_out, int32_t nthreads) {
    parallel_for(T, nthreads, [&](int64_t t) {
        std::vector<double> zl(E);
        double* z = z_out ? z_out + t * E : zl.data();
        logits_token(x + t * d, Wr, d, E, z);
        Route r = route_token(z, bias, E, G, KG, K, S, norm);
        for (int j = 0; j < K; ++j) {
            idx_out[t * K + j] = r.idx[j];
            w_out[t * K + j] = r.w[j];
        }
        gap_out[t] = r.gap;
    });
}

// Routing weights for a given selection idx [T,K] (used when a token's selection is excused).
void oracle_weights_for(const double* z, int64_t T, int32_t E, int32_t K, const int32_t* idx, double S,
                        int32_t norm, double* w_out) {
    for (int64_t t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int j = 0; j < K; ++j) sum += sigmoid(z[t * E + idx[t * K + j]]);
        for (int j = 0; j < K; ++j) {
            double s = sigmoid(z[t * E + idx[t * K + j]]);
            w_out[t * K + j] = norm ? S * s / sum : S * s;
        }
    }
}

// Token -> expert dispatch: pairs p = t*K + j ordered by expert id, stably.
// offsets [E+1], sorted_pairs [P], pair_rank [P] (position of pair p in sorted order).
void oracle_dispatch(const int32_t* idx, int64_t P, int32_t E, int32_t* offsets, int32_t* sorted_pairs,
                     int32_t* pair_rank) {
    std::vector<int32_t> order(P);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t c) { return idx[a] < idx[c]; });
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) offsets[idx[p] + 1] += 1;
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int64_t i = 0; i < P; ++i) {
        sorted_pairs[i] = order[i];
        pair_rank[order[i]] = (int32_t)i;
    }
}

// One expert on n token rows: o [n,d] (double), with the bf16 rounding of h.
void oracle_expert(const uint16_t* x_rows, int64_t n, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                   int32_t d, int32_t I, double* o_out, int32_t nthreads) {
    parallel_for(n, nthreads, [&](int64_t i) { expert_token(x_rows + i * d, wg, wu, wd, d, I, o_out + i * d); });
}

// Layer output for n token rows given their routing: y[i] = sum_j w[i,j] * expert_{idx[i,j]}(x[i]).
// Expert weights are passed per expert id (arrays of E pointers; unused entries may be NULL).
void oracle_moe_rows(const uint16_t* x_rows, int64_t n, const int32_t* idx, const double* w, int32_t K,
                     const uint16_t* const* wg, const uint16_t* const* wu, const uint16_t* const* wd,
                     int32_t d, int32_t I, double* y_out, int32_t nthreads) {
    int64_t work = n * K;
    std::vector<double> o((size_t)work * d);
    parallel_for(work, nthreads, [&](int64_t q) {
        int64_t i = q / K;
        int e = idx[q];
        expert_token(x_rows + i * d, wg[e], wu[e], wd[e], d, I, o.data() + q * d);
    });
    for (int64_t i = 0; i < n; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) acc += w[i * K + j] * o[(i * K + j) * d + c];
            y_out[i * d + c] = acc;
        }
}


// Expert-parallel share ("Use HF Transformers" cookbook, Parallelism: each GPU holds a
// contiguous block of the experts and computes the tokens routed to them): the part of
// the layer output that experts [e_begin, e_begin + e_count) contribute,
// y_part[i] = sum over slots j with idx[i,j] in that range, in slot order, of
// w[i,j] * expert(x_i). Slots outside the range add nothing; a row with none is 0.
// wg/wu/wd are indexed by the local id idx - e_begin. Summed over a partition of the
// experts into such ranges, the shares give the whole layer output.
void oracle_moe_share_rows(const uint16_t* x_rows, int64_t n, const int32_t* idx, const double* w, int32_t K,
                           int32_t e_begin, int32_t e_count, const uint16_t* const* wg, const uint16_t* const* wu,
                           const uint16_t* const* wd, int32_t d, int32_t I, double* y_out, int32_t nthreads) {
    auto local = [&](int64_t q) {
        const int e = idx[q] - e_begin;
        return (e >= 0 && e < e_count) ? e : -1;
    };
    int64_t work = n * K;
    std::vector<double> o((size_t)work * d, 0.0);
    parallel_for(work, nthreads, [&](int64_t q) {
        const int e = local(q);
        if (e >= 0) expert_token(x_rows + (q / K) * d, wg[e], wu[e], wd[e], d, I, o.data() + q * d);
    });
    for (int64_t i = 0; i < n; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j)
                if (local(i * K + j) >= 0) acc += w[i * K + j] * o[(i * K + j) * d + c];
            y_out[i * d + c] = acc;
        }
}

// Post-MLP RMSNorm of the layer output y [T,d] (double, unrounded): n[t,j] = y[t,j] * r_t * w[j],
// r_t = 1 / sqrt(mean_j y[t,j]^2 + eps).
void oracle_post_norm(const double* y, const uint16_t* w, int64_t T, int32_t d, double eps, double* n_out,
                      int32_t nthreads) {
    parallel_for(T, nthreads, [&](int64_t t) {
        const double* yr = y + t * d;
        double ss = 0.0;
        for (int j = 0; j < d; ++j) ss += yr[j] * yr[j];
        double r = 1.0 / std::sqrt(ss / d + eps);
        for (int j = 0; j < d; ++j) n_out[t * d + j] = yr[j] * r * bf16_value(w[j]);
    });
}

// Depth-scaled residual add of the k-th contribution c to the stream r (k >= 1):
// r_out = r * sqrt((k-1)/k) + c / sqrt(k). After contributions c_1..c_m added with
// k = 1..m the stream is (c_1 + ... + c_m) / sqrt(m).
void oracle_residual_step(const double* r, const double* c, int64_t n, int32_t k, double* r_out) {
    const double keep = std::sqrt((double)(k - 1) / (double)k);
    const double add = 1.0 / std::sqrt((double)k);
    for (int64_t i = 0; i < n; ++i) r_out[i] = r[i] * keep + c[i] * add;
}

// Position of a sublayer's output among the residual contributions: the embedding is the
// first, then attention and MLP of each layer in turn (0-indexed layer i: attention 2(i+1),
// MLP 2(i+1)+1).
int32_t oracle_contribution_index(int32_t layer, int32_t is_mlp) { return 2 * (layer + 1) + (is_mlp ? 1 : 0); }


// ---- FP8 (OCP E4M3) weights with one power-of-two scale per 32 values (OCP MX) ----------

// Value of an E4M3 code: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
// holds the subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN.
double oracle_e4m3_value(uint8_t c) {
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return std::nan("");
    if (e == 0) v = std::ldexp((double)m, -9);
    else v = std::ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

// Nearest E4M3 code to v, ties to the even mantissa, magnitudes at or above 448 saturated.
uint8_t oracle_e4m3_round(double v) {
    const uint8_t sgn = std::signbit(v) ? 0x80 : 0x00;
    const double a = std::fabs(v);
    if (a >= 448.0) return sgn | 0x7E;
    int ex;
    std::frexp(a, &ex);          // a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    int e = ex - 1;
    if (a == 0.0 || e < -6) {    // subnormal range: multiples of 2^-9
        const int m = (int)std::nearbyint(std::ldexp(a, 9));
        return sgn | (uint8_t)m; // m == 8 is the code of 2^-6, the smallest normal
    }
    int m = (int)std::nearbyint((std::ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8) {
        m = 0;
        ++e;
    }
    return sgn | (uint8_t)(((e + 7) << 3) | m);
}

// Quantize a [rows, K] bf16 matrix (K % 32 == 0) into E4M3 codes q [rows, K] and E8M0 scale
// bytes s [rows, K/32]: block b of row r holds 2^(s - 127) * e4m3(q).
void oracle_fp8_quantize(const uint16_t* w, int64_t rows, int32_t K, uint8_t* q, uint8_t* s, int32_t nthreads) {
    const int nb = K / 32;
    parallel_for(rows, nthreads, [&](int64_t r) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t* blk = w + r * K + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(bf16_value(blk[i])));
            int shared = 0;
            if (amax > 0.0) {
                int ex;
                std::frexp(amax, &ex);
                shared = std::min(127, std::max(-127, (ex - 1) - 8));
            }
            s[r * nb + b] = (uint8_t)(shared + 127);
            for (int i = 0; i < 32; ++i) q[r * K + 32 * b + i] = oracle_e4m3_round(std::ldexp(bf16_value(blk[i]), -shared));
        }
    });
}

// Dequantize back to bf16 bits (the products are exact in bf16 for every scale >= 2^-118,
// i.e. any trained weight); returns the number of elements that were not exact.
int64_t oracle_fp8_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int32_t K, uint16_t* out) {
    const int nb = K / 32;
    int64_t inexact = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int k = 0; k < K; ++k) {
            const double v = std::ldexp(oracle_e4m3_value(q[r * K + k]), (int)s[r * nb + k / 32] - 127);
            const uint16_t b = bf16_round(v);
            if (bf16_value(b) != v) ++inexact;
            out[r * K + k] = b;
        }
    return inexact;
}

}  // extern "C"
