// C ABI of libbeam_moe.so: argument validation, workspace carving and kernel launches
// on the caller's stream. Contract and citations: include/beam_moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/beam_moe.h"
#include "kernels.h"

namespace {

using beam::Shape;

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

beam_moe_status to_shape(const beam_moe_shape* p, Shape* s) {
    if (!p) return BEAM_MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->d <= 0 || p->E <= 0 || p->n_group <= 0 || p->topk_group <= 0 || p->top_k <= 0 || p->I <= 0)
        return BEAM_MOE_ERR_INVALID_ARG;
    if (!std::isfinite(p->routed_scaling_factor) || !std::isfinite(p->rms_eps) || p->rms_eps < 0.0f)
        return BEAM_MOE_ERR_INVALID_ARG;
    if (p->E % p->n_group != 0 || p->topk_group > p->n_group) return BEAM_MOE_ERR_INVALID_ARG;
    const int gsz = p->E / p->n_group;
    if (p->top_k > p->topk_group * gsz) return BEAM_MOE_ERR_INVALID_ARG;
    if (p->d % 64 || p->I % 64 || p->top_k > 16 || p->n_group > 64 || gsz < 2) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    int epl = 1;
    if (p->E > 64) {
        if (p->E != 128 && p->E != 256 && p->E != 512 && p->E != 1024) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
        epl = p->E / 64;
    }
    if (gsz % epl || !pow2(gsz / epl)) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    if (p->T * (int64_t)p->top_k >= (int64_t)INT32_MAX) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    if (p->weight_layout != BEAM_MOE_WEIGHTS_ROW_MAJOR && p->weight_layout != BEAM_MOE_WEIGHTS_PACKED)
        return BEAM_MOE_ERR_INVALID_ARG;
    s->T = p->T; s->d = p->d; s->E = p->E; s->G = p->n_group; s->KG = p->topk_group; s->K = p->top_k; s->I = p->I;
    s->S = p->routed_scaling_factor; s->norm = p->norm_topk_prob ? 1 : 0; s->eps = p->rms_eps;
    s->packed = p->weight_layout == BEAM_MOE_WEIGHTS_PACKED ? 1 : 0;
    s->route_E = p->E;
    return BEAM_MOE_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace segments, each 256-byte aligned.
struct Layout {
    size_t xn, wrs, zp, idx, w, cc, ric, off, sp, pr, tiles, ntiles, h, yp, total;
};

Layout layout(const Shape& s) {
    const size_t T = (size_t)s.T, P = T * s.K;
    const size_t n_chunks = (P + beam::kChunkPairs - 1) / beam::kChunkPairs;
    const size_t max_tiles = (P + 15) / 16 + (size_t)s.E;
    Layout L{};
    size_t o = 0;
    L.xn = o; o += up(T * s.d * 2);
    L.wrs = o; o += up(beam::router_split_bytes(s));
    L.zp = o; o += up(beam::router_zp_floats(s) * 4);
    L.idx = o; o += up(P * 4);
    L.w = o; o += up(P * 4);
    L.cc = o; o += up(n_chunks * s.E * 4);
    L.ric = o; o += up(P * 4);
    L.off = o; o += up(((size_t)s.E + 1) * 4);
    L.sp = o; o += up(P * 4);
    L.pr = o; o += up(P * 4);
    L.tiles = o; o += up(max_tiles * 4 * 4);
    L.ntiles = o; o += up(beam::kTileWords * 4);
    L.h = o; o += up(P * s.I * 2);
    L.yp = o; o += up(P * s.d * 4);
    L.total = o;
    return L;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

beam_moe_status hip_status() { return hipGetLastError() == hipSuccess ? BEAM_MOE_OK : BEAM_MOE_ERR_HIP; }

// Router into caller-visible buffers; with a norm weight the router norms x into x_normed first.
void run_route(const Shape& s, const Layout& L, const void* x, const void* norm_w, void* x_normed, const float* Wr,
               const float* bias, int32_t* idx, float* w, float* logits, void* ws, hipStream_t st) {
    beam::launch_router(s, x, norm_w, x_normed, Wr, bias, at<void>(ws, L.wrs), at<float>(ws, L.zp), idx, w, logits,
                        st);
}

}  // namespace

extern "C" {

size_t beam_moe_workspace_bytes(const beam_moe_shape* shape) {
    Shape s;
    if (to_shape(shape, &s) != BEAM_MOE_OK) return 0;
    return layout(s).total;
}

beam_moe_status beam_moe_route(const beam_moe_shape* shape, const void* x, const void* norm_w, void* x_normed,
                               const float* Wr, const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                               void* workspace, size_t ws_bytes, void* stream) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    if (!x || !Wr || !bias || !topk_idx || !topk_w || (norm_w && !x_normed)) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(Wr) || !aligned(bias) || !aligned(topk_idx) || !aligned(topk_w) ||
        (norm_w && (!aligned(norm_w) || !aligned(x_normed))) || (logits && !aligned(logits)))
        return BEAM_MOE_ERR_INVALID_ARG;
    if (s.T == 0) return BEAM_MOE_OK;
    const Layout L = layout(s);
    if (!workspace || !aligned(workspace)) return BEAM_MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    (void)hipGetLastError();
    run_route(s, L, x, norm_w, x_normed, Wr, bias, topk_idx, topk_w, logits, workspace, (hipStream_t)stream);
    return hip_status();
}

beam_moe_status beam_moe_dispatch(const beam_moe_shape* shape, const int32_t* topk_idx, int32_t* expert_offsets,
                                  int32_t* sorted_pairs, int32_t* pair_rank, void* workspace, size_t ws_bytes,
                                  void* stream) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    if (!topk_idx || !expert_offsets || !sorted_pairs) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(topk_idx) || !aligned(expert_offsets) || !aligned(sorted_pairs) || (pair_rank && !aligned(pair_rank)))
        return BEAM_MOE_ERR_INVALID_ARG;
    if (s.T == 0) return BEAM_MOE_OK;
    const Layout L = layout(s);
    if (!workspace || !aligned(workspace)) return BEAM_MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    (void)hipGetLastError();
    beam::launch_dispatch(s, topk_idx, expert_offsets, sorted_pairs, pair_rank, at<int32_t>(workspace, L.cc),
                          at<int32_t>(workspace, L.ric), nullptr, nullptr, 16, (hipStream_t)stream);
    return hip_status();
}

}  // extern "C"

namespace {

// Optional post-MLP norm + depth-scaled residual applied in the combine.
struct Post {
    const void* w = nullptr;
    int layer = 0;
    const float* resid = nullptr;
    float* resid_out = nullptr;
};

// Optional FP8 expert weights (decode-sized batches): codes and per-32 scale bytes.
struct Fp8 {
    const void *Wg, *Wu, *Wd, *sg, *su, *sd;
};

beam_moe_status check_fp8(const Shape& s, const Fp8& f) {
    if (!f.Wg || !f.Wu || !f.Wd || !f.sg || !f.su || !f.sd) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(f.Wg) || !aligned(f.Wu) || !aligned(f.Wd) || !aligned(f.sg) || !aligned(f.su) || !aligned(f.sd))
        return BEAM_MOE_ERR_INVALID_ARG;
    if (!beam::fp8_supports(s)) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    return BEAM_MOE_OK;
}

beam_moe_status check_post(const Shape& s, const Post& p) {
    if (!p.w || !p.resid || !p.resid_out || p.layer < 0) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(p.w) || !aligned(p.resid) || !aligned(p.resid_out)) return BEAM_MOE_ERR_INVALID_ARG;
    if (s.d > beam::kPostMaxD) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    return BEAM_MOE_OK;
}

// The layer's tensor arguments: required ones present, all 16-byte aligned (y may be absent when
// the post-MLP residual takes the output).
beam_moe_status check_tensors(const void* x, const void* norm_w, const float* Wr, const float* bias, const void* Wg,
                              const void* Wu, const void* Wd, const float* y, const int32_t* topk_idx,
                              const float* topk_w, const float* logits, bool post) {
    if (!x || !Wr || !bias || !Wg || !Wu || !Wd || (!y && !post)) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(Wr) || !aligned(bias) || !aligned(Wg) || !aligned(Wu) || !aligned(Wd) ||
        (y && !aligned(y)) || (norm_w && !aligned(norm_w)) || (topk_idx && !aligned(topk_idx)) ||
        (topk_w && !aligned(topk_w)) || (logits && !aligned(logits)))
        return BEAM_MOE_ERR_INVALID_ARG;
    return BEAM_MOE_OK;
}

beam_moe_status forward_impl(const beam_moe_shape* shape, const void* x, const void* norm_w, const float* Wr,
                             const float* bias, const void* Wg, const void* Wu, const void* Wd, float* y,
                             int32_t* topk_idx, float* topk_w, float* logits, void* workspace, size_t ws_bytes,
                             void* stream, void* const* events, const Post* post, const Fp8* fp8 = nullptr) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    if (fp8) {
        if ((st = check_fp8(s, *fp8)) != BEAM_MOE_OK) return st;
        Wg = fp8->Wg;
        Wu = fp8->Wu;
        Wd = fp8->Wd;
    }
    if ((st = check_tensors(x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, post != nullptr)) !=
        BEAM_MOE_OK)
        return st;
    if (post && (st = check_post(s, *post)) != BEAM_MOE_OK) return st;
    if (s.T == 0) return BEAM_MOE_OK;
    const Layout L = layout(s);
    if (!workspace || !aligned(workspace)) return BEAM_MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    auto mark = [&](int i) {
        if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], hs);
    };
    int32_t* idx = topk_idx ? topk_idx : at<int32_t>(workspace, L.idx);
    float* w = topk_w ? topk_w : at<float>(workspace, L.w);
    void* xn = at<void>(workspace, L.xn);
    mark(0);
    run_route(s, L, x, norm_w, xn, Wr, bias, idx, w, logits, workspace, hs);
    mark(1);
    const void* xin = norm_w ? xn : x;
    int32_t* off = at<int32_t>(workspace, L.off);
    int32_t* sp = at<int32_t>(workspace, L.sp);
    int32_t* pr = at<int32_t>(workspace, L.pr);
    int32_t* tiles = at<int32_t>(workspace, L.tiles);
    int32_t* ntiles = at<int32_t>(workspace, L.ntiles);
    // the tile list feeds only the tiled GEMMs; the weight streams read the offsets alone
    const bool tiled = !fp8 && beam::experts_tiled(s);
    beam::launch_dispatch(s, idx, off, sp, pr, at<int32_t>(workspace, L.cc), at<int32_t>(workspace, L.ric),
                          tiled ? tiles : nullptr, ntiles, beam::experts_tile_m(s), hs);
    mark(2);
    void* h = at<void>(workspace, L.h);
    float* yp = at<float>(workspace, L.yp);
    if (fp8)
        beam::launch_swiglu_fp8(s, xin, off, sp, fp8->Wg, fp8->Wu, fp8->sg, fp8->su, h, hs);
    else
        beam::launch_swiglu(s, xin, off, sp, tiles, ntiles, Wg, Wu, h, hs);
    mark(3);
    if (fp8)
        beam::launch_down_fp8(s, h, off, fp8->Wd, fp8->sd, yp, hs);
    else
        beam::launch_down(s, h, off, sp, tiles, ntiles, Wd, yp, hs);
    mark(4);
    if (post)
        beam::launch_combine_post_residual(s, yp, pr, w, post->w, post->layer, post->resid, post->resid_out, y, hs);
    else
        beam::launch_combine(s, yp, pr, w, y, hs);
    mark(5);
    return hip_status();
}

}  // namespace

extern "C" {

beam_moe_status beam_moe_forward(const beam_moe_shape* shape, const void* x, const void* norm_w, const float* Wr,
                                 const float* bias, const void* Wg, const void* Wu, const void* Wd, float* y,
                                 int32_t* topk_idx, float* topk_w, float* logits, void* workspace, size_t ws_bytes,
                                 void* stream) {
    return forward_impl(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, workspace, ws_bytes,
                        stream, nullptr, nullptr);
}

beam_moe_status beam_moe_forward_staged(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                        const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                        const void* Wd, float* y, int32_t* topk_idx, float* topk_w, float* logits,
                                        void* workspace, size_t ws_bytes, void* stream, void* const* stage_events) {
    return forward_impl(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, workspace, ws_bytes,
                        stream, stage_events, nullptr);
}

beam_moe_status beam_moe_forward_residual(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                          const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                          const void* Wd, const void* post_w, int32_t layer, const float* resid,
                                          float* resid_out, float* y, int32_t* topk_idx, float* topk_w,
                                          float* logits, void* workspace, size_t ws_bytes, void* stream,
                                          void* const* stage_events) {
    Post p;
    p.w = post_w;
    p.layer = layer;
    p.resid = resid;
    p.resid_out = resid_out;
    return forward_impl(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, workspace, ws_bytes,
                        stream, stage_events, &p);
}

beam_moe_status beam_moe_post_residual(const beam_moe_shape* shape, const float* y, const void* post_w, int32_t layer,
                                       const float* resid, float* resid_out, void* stream) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    Post p;
    p.w = post_w;
    p.layer = layer;
    p.resid = resid;
    p.resid_out = resid_out;
    if (!y || !aligned(y)) return BEAM_MOE_ERR_INVALID_ARG;
    if ((st = check_post(s, p)) != BEAM_MOE_OK) return st;
    if (s.T == 0) return BEAM_MOE_OK;
    (void)hipGetLastError();
    beam::launch_post_residual(s, y, post_w, layer, resid, resid_out, (hipStream_t)stream);
    return hip_status();
}

beam_moe_status beam_moe_quantize_fp8(int64_t rows, int32_t K, const void* w, void* q, void* scales, void* stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return BEAM_MOE_ERR_INVALID_ARG;
    if (!w || !q || !scales || !aligned(w) || !aligned(q)) return BEAM_MOE_ERR_INVALID_ARG;
    if (rows * (int64_t)K >= ((int64_t)1 << 40)) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    if (rows == 0) return BEAM_MOE_OK;
    (void)hipGetLastError();
    beam::launch_fp8_quantize(rows, K, w, q, scales, (hipStream_t)stream);
    return hip_status();
}

beam_moe_status beam_moe_forward_fp8(const beam_moe_shape* shape, const void* x, const void* norm_w, const float* Wr,
                                     const float* bias, const void* Wg8, const void* Wu8, const void* Wd8,
                                     const void* sg, const void* su, const void* sd, float* y, int32_t* topk_idx,
                                     float* topk_w, float* logits, void* workspace, size_t ws_bytes, void* stream,
                                     void* const* stage_events) {
    Fp8 f{Wg8, Wu8, Wd8, sg, su, sd};
    return forward_impl(shape, x, norm_w, Wr, bias, nullptr, nullptr, nullptr, y, topk_idx, topk_w, logits, workspace,
                        ws_bytes, stream, stage_events, nullptr, &f);
}

constexpr int32_t kDenseMinI = 2048;

size_t beam_moe_dense_workspace_bytes(int64_t T, int32_t d, int32_t I) {
    if (T < 0 || d <= 0 || I <= 0) return 0;
    size_t n = up((size_t)T * (size_t)I * 2);
    if (beam::dense_stream_supports(T, d, I)) n = std::max(n, beam::dense_stream_workspace_bytes(T, d, I));
    return n;
}

beam_moe_status beam_moe_dense_mlp(int64_t T, int32_t d, int32_t I, int32_t weight_layout, const void* x,
                                   const void* Wg, const void* Wu, const void* Wd, float* y, void* workspace,
                                   size_t ws_bytes, void* stream) {
    if (T < 0 || d <= 0 || I <= 0) return BEAM_MOE_ERR_INVALID_ARG;
    if (weight_layout != BEAM_MOE_WEIGHTS_ROW_MAJOR && weight_layout != BEAM_MOE_WEIGHTS_PACKED)
        return BEAM_MOE_ERR_INVALID_ARG;
    if (!x || !Wg || !Wu || !Wd || !y) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(Wg) || !aligned(Wu) || !aligned(Wd) || !aligned(y)) return BEAM_MOE_ERR_INVALID_ARG;
    const int64_t lim = (int64_t)1 << 31;
    if (T * (int64_t)d >= lim || T * (int64_t)I >= lim || (int64_t)d * I >= lim) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    // the output bar (max|dy| <= 1e-2 rms(y)) holds only from I = 2048: one bf16 ulp of one large h
    // element, rounded from FP32 rather than FP64 sums, moves y by ~2^-4 * 3.5 / sqrt(I) ~ 1e-2 rms(y)
    // at I = 512
    if (I < kDenseMinI) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    const bool stream_path = beam::dense_stream_supports(T, d, I);
    if (!stream_path && !beam::dense_supports(T, d, I)) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    if (T == 0) return BEAM_MOE_OK;
    if (!workspace || !aligned(workspace)) return BEAM_MOE_ERR_INVALID_ARG;
    if (ws_bytes < beam_moe_dense_workspace_bytes(T, d, I)) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t hs = (hipStream_t)stream;
    const bool packed = weight_layout == BEAM_MOE_WEIGHTS_PACKED;
    (void)hipGetLastError();
    if (stream_path) {
        beam::launch_dense_stream(T, d, I, packed, x, Wg, Wu, Wd, y, workspace, hs);
    } else {
        beam::launch_dense_swiglu(T, d, I, packed, x, Wg, Wu, workspace, hs);
        beam::launch_dense_down(T, d, I, packed, workspace, Wd, y, hs);
    }
    return hip_status();
}

size_t beam_moe_share_workspace_bytes(const beam_moe_shape* shape, int32_t e_count) {
    Shape s;
    if (to_shape(shape, &s) != BEAM_MOE_OK || e_count < 1 || e_count > s.E) return 0;
    Shape sl = s;
    sl.E = e_count;
    return layout(sl).total;
}

beam_moe_status beam_moe_experts_share(const beam_moe_shape* shape, int32_t e_begin, int32_t e_count, const void* x,
                                       const int32_t* topk_idx, const float* topk_w, const void* Wg, const void* Wu,
                                       const void* Wd, float* y_part, void* workspace, size_t ws_bytes, void* stream,
                                       void* const* stage_events) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    if (e_count < 1 || e_begin < 0 || e_begin > s.E - e_count) return BEAM_MOE_ERR_INVALID_ARG;
    if (!x || !topk_idx || !topk_w || !Wg || !Wu || !Wd || !y_part) return BEAM_MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(topk_idx) || !aligned(topk_w) || !aligned(Wg) || !aligned(Wu) || !aligned(Wd) ||
        !aligned(y_part))
        return BEAM_MOE_ERR_INVALID_ARG;
    if (s.T == 0) return BEAM_MOE_OK;
    Shape sl = s;                 // the local experts are the whole expert set of this call;
    sl.E = e_count;               // the path (streams or tiled GEMM) is still chosen on all E
    const Layout L = layout(sl);
    if (!workspace || !aligned(workspace)) return BEAM_MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    auto mark = [&](int i) {
        if (stage_events && stage_events[i]) (void)hipEventRecord((hipEvent_t)stage_events[i], hs);
    };
    int32_t* idl = at<int32_t>(workspace, L.idx);
    int32_t* off = at<int32_t>(workspace, L.off);
    int32_t* sp = at<int32_t>(workspace, L.sp);
    int32_t* pr = at<int32_t>(workspace, L.pr);
    int32_t* tiles = at<int32_t>(workspace, L.tiles);
    int32_t* ntiles = at<int32_t>(workspace, L.ntiles);
    void* h = at<void>(workspace, L.h);
    float* yp = at<float>(workspace, L.yp);
    mark(0);
    mark(1);
    beam::launch_share_idx(topk_idx, s.T * s.K, e_begin, e_count, idl, hs);
    beam::launch_dispatch(sl, idl, off, sp, pr, at<int32_t>(workspace, L.cc), at<int32_t>(workspace, L.ric),
                          beam::experts_tiled(sl) ? tiles : nullptr, ntiles, beam::experts_tile_m(sl), hs);
    mark(2);
    beam::launch_swiglu(sl, x, off, sp, tiles, ntiles, Wg, Wu, h, hs);
    mark(3);
    beam::launch_down(sl, h, off, sp, tiles, ntiles, Wd, yp, hs);
    mark(4);
    beam::launch_combine(sl, yp, pr, topk_w, y_part, hs);
    mark(5);
    return hip_status();
}

beam_moe_status beam_moe_pack_weights(int64_t rows, int32_t K, const void* w, void* packed, void* stream) {
    if (rows < 0 || rows % 16 != 0 || K <= 0 || K % 32 != 0) return BEAM_MOE_ERR_INVALID_ARG;
    if (!w || !packed || !aligned(w) || !aligned(packed) || w == packed) return BEAM_MOE_ERR_INVALID_ARG;
    if (rows * (int64_t)K >= ((int64_t)1 << 40)) return BEAM_MOE_ERR_UNSUPPORTED_SHAPE;
    if (rows == 0) return BEAM_MOE_OK;
    (void)hipGetLastError();
    beam::launch_pack_stream(w, packed, rows, K, (hipStream_t)stream);
    return hip_status();
}

}  // extern "C"

// Scratch of beam_moe_forward_noalloc: the layer's workspace for callers that cannot allocate.
// Each GPU the library runs on holds its own copy until the process ends. Host code never uses
// the array's name as an address: the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

beam_moe_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BEAM_MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_MOE_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return BEAM_MOE_OK;
}

}  // namespace

extern "C" {

beam_moe_status beam_moe_forward_noalloc(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                         const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                         const void* Wd, float* y, int32_t* topk_idx, float* topk_w, float* logits,
                                         void* stream) {
    Shape s;
    beam_moe_status st = to_shape(shape, &s);
    if (st != BEAM_MOE_OK) return st;
    if ((st = check_tensors(x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, false)) != BEAM_MOE_OK)
        return st;
    if (s.T == 0) return BEAM_MOE_OK;
    if (layout(s).total > kScratchBytes) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != BEAM_MOE_OK) return st;
    // nothing in the scratch has to start at zero: the dispatch zeroes its own counters on every call
    return forward_impl(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, ws, kScratchBytes,
                        stream, nullptr, nullptr);
}

const char* beam_moe_status_string(int32_t status) {
    switch (status) {
        case BEAM_MOE_OK: return "ok";
        case BEAM_MOE_ERR_INVALID_ARG: return "invalid argument";
        case BEAM_MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case BEAM_MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case BEAM_MOE_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

}  // extern "C"
