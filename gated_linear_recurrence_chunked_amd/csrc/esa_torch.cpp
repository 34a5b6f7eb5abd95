// The library's calls from Python without ctypes: torch tensors in, the C ABI out.
// Argument marshalling only: the checks the Python binding documents (shapes, dtypes,
// devices, layouts), output allocation, the current HIP stream of the tensors' device; the
// computation is the library's kernels behind esa_scan_fwd, esa_scan_bwd, esa_state_step
// and the sequence-segment calls.  Through ctypes with the checks in Python a call cost 10 us (forward),
// 17 us (backward) and 5-7 us (decode step) of host time, more than the kernels of small
// problems take; here it is a few microseconds.
//
// Errors in the arguments raise TypeError or ValueError before anything is launched; a
// status the library returns is handed back to the caller, which raises its own error type.
#include <torch/extension.h>

#include <c10/hip/HIPGuard.h>
#include <c10/hip/HIPStream.h>

#include <algorithm>
#include <tuple>

#include "esa.h"

namespace {

int dtype_code(at::ScalarType t) {
    switch (t) {
        case at::kFloat: return ESA_F32;
        case at::kHalf: return ESA_F16;
        case at::kBFloat16: return ESA_BF16;
        case at::kFloat8_e4m3fn: return ESA_F8E4M3;
        case at::kFloat8_e5m2: return ESA_F8E5M2;
        default: return -1;
    }
}

// A sequence input [B, T, H, Dh]: a CUDA (HIP) tensor of a storage dtype; `like` (the gate
// logits) fixes shape, dtype and device for the others.  Returns it contiguous.
at::Tensor seq(const char* name, const at::Tensor& t, const at::Tensor* like) {
    TORCH_CHECK_TYPE(t.is_cuda(), name, " must be a CUDA (HIP) tensor");
    TORCH_CHECK_VALUE(t.dim() == 4, name, " must be [B, T, H, Dh], got ", t.sizes());
    TORCH_CHECK_TYPE(dtype_code(t.scalar_type()) >= 0, name, ": dtype ", t.scalar_type(),
                     " not supported");
    if (like)
        TORCH_CHECK_VALUE(t.sizes() == like->sizes() && t.scalar_type() == like->scalar_type() &&
                              t.device() == like->device(),
                          name, " must match shape/dtype/device of the gate logits");
    return t.contiguous();
}

// An optional fp32 state [B, H, Dh] on the inputs' device; returned contiguous.
c10::optional<at::Tensor> state(const char* name, const c10::optional<at::Tensor>& t,
                                at::IntArrayRef shape, const c10::Device& dev) {
    if (!t.has_value()) return c10::nullopt;
    TORCH_CHECK_VALUE(t->scalar_type() == at::kFloat && t->sizes() == shape && t->device() == dev,
                      name, " must be fp32 ", shape, " on ", dev);
    return t->contiguous();
}

// A caller-provided output is written in place, so it must already be what the library
// writes: contiguous, of the given shape, dtype and device (no copy is made).
void out(const char* name, const at::Tensor& t, at::IntArrayRef shape, at::ScalarType dt,
         const c10::Device& dev) {
    TORCH_CHECK_VALUE(t.sizes() == shape && t.scalar_type() == dt && t.device() == dev &&
                          t.is_contiguous(),
                      name, " must be a contiguous ", dt, " tensor of shape ", shape, " on ", dev);
}

const void* ptr(const c10::optional<at::Tensor>& t) { return t.has_value() ? t->data_ptr() : nullptr; }

// The workspace (any dtype; its bytes count) must be device memory of the inputs' device.
void check_workspace(const at::Tensor& ws, const c10::Device& dev) {
    TORCH_CHECK_VALUE(ws.device() == dev && ws.is_contiguous(),
                      "workspace must be a contiguous tensor on ", dev);
}

// esa_scan_fwd.  Returns (status, y, final_state, ckpt or None).
std::tuple<int64_t, at::Tensor, at::Tensor, c10::optional<at::Tensor>> scan_fwd(
    const at::Tensor& a_, const at::Tensor& v_, const at::Tensor& q_,
    const c10::optional<at::Tensor>& init_state_, int64_t mode, bool return_ckpt,
    c10::optional<at::Tensor> final_state, c10::optional<at::Tensor> y, at::Tensor workspace) {
    const at::Tensor a = seq("gate_logit", a_, nullptr);
    const at::Tensor v = seq("value", v_, &a);
    const at::Tensor q = seq("query", q_, &a);
    const int64_t B = a.size(0), T = a.size(1), H = a.size(2), Dh = a.size(3);
    const c10::Device dev = a.device();
    const std::vector<int64_t> sshape{B, H, Dh};
    const auto init_state = state("init_state", init_state_, sshape, dev);
    if (y.has_value())
        out("y", *y, a.sizes(), a.scalar_type(), dev);
    else
        y = at::empty_like(a);
    if (final_state.has_value())
        out("final_state", *final_state, sshape, at::kFloat, dev);
    else
        final_state = at::empty(sshape, a.options().dtype(at::kFloat));
    check_workspace(workspace, dev);
    c10::optional<at::Tensor> ckpt;
    if (return_ckpt) {
        const int64_t n = std::max<int64_t>(1, (int64_t)(esa_scan_ckpt_bytes(B, T, H, Dh) / 4));
        ckpt = at::empty({n}, a.options().dtype(at::kFloat));
    }
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t s = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int st = esa_scan_fwd(B, T, H, Dh, dtype_code(a.scalar_type()), (int)mode, a.data_ptr(),
                                v.data_ptr(), q.data_ptr(), static_cast<const float*>(ptr(init_state)),
                                y->data_ptr(), final_state->data_ptr<float>(),
                                ckpt.has_value() ? ckpt->data_ptr<float>() : nullptr,
                                workspace.data_ptr(), workspace.nbytes(), s);
    return {st, *y, *final_state, ckpt};
}

// esa_scan_bwd.  Returns (status, d_logit, d_value, d_query, d_init).
std::tuple<int64_t, at::Tensor, at::Tensor, at::Tensor, at::Tensor> scan_bwd(
    const at::Tensor& a_, const at::Tensor& v_, const at::Tensor& q_, const at::Tensor& dy_,
    const c10::optional<at::Tensor>& init_state_, const c10::optional<at::Tensor>& d_final_,
    const c10::optional<at::Tensor>& ckpt_, int64_t mode, at::Tensor workspace,
    c10::optional<at::Tensor> da, c10::optional<at::Tensor> dv, c10::optional<at::Tensor> dq,
    c10::optional<at::Tensor> d_init) {
    const at::Tensor a = seq("gate_logit", a_, nullptr);
    const at::Tensor v = seq("value", v_, &a);
    const at::Tensor q = seq("query", q_, &a);
    const at::Tensor dy = seq("dy", dy_, &a);
    const int64_t B = a.size(0), T = a.size(1), H = a.size(2), Dh = a.size(3);
    const c10::Device dev = a.device();
    const std::vector<int64_t> sshape{B, H, Dh};
    const auto init_state = state("init_state", init_state_, sshape, dev);
    const auto d_final = state("d_final_state", d_final_, sshape, dev);
    check_workspace(workspace, dev);
    c10::optional<at::Tensor> ckpt;
    if (ckpt_.has_value()) {
        TORCH_CHECK_VALUE(ckpt_->scalar_type() == at::kFloat && ckpt_->device() == dev &&
                              (size_t)ckpt_->numel() * 4 >= esa_scan_ckpt_bytes(B, T, H, Dh),
                          "ckpt must be the fp32 checkpoint of scan_fwd(return_ckpt=True)");
        ckpt = ckpt_->contiguous();
    }
    const char* names[3] = {"d_logit", "d_value", "d_query"};
    c10::optional<at::Tensor>* grads[3] = {&da, &dv, &dq};
    for (int k = 0; k < 3; ++k) {
        if (grads[k]->has_value())
            out(names[k], **grads[k], a.sizes(), a.scalar_type(), dev);
        else
            *grads[k] = at::empty_like(a);
    }
    if (d_init.has_value())
        out("d_init", *d_init, sshape, at::kFloat, dev);
    else
        d_init = at::empty(sshape, a.options().dtype(at::kFloat));
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t s = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int st = esa_scan_bwd(B, T, H, Dh, dtype_code(a.scalar_type()), (int)mode, a.data_ptr(),
                                v.data_ptr(), q.data_ptr(), static_cast<const float*>(ptr(init_state)),
                                dy.data_ptr(), static_cast<const float*>(ptr(d_final)),
                                static_cast<const float*>(ptr(ckpt)), da->data_ptr(), dv->data_ptr(),
                                dq->data_ptr(), d_init->data_ptr<float>(), workspace.data_ptr(),
                                workspace.nbytes(), s);
    return {st, *da, *dv, *dq, *d_init};
}

// esa_scan_segment_fwd.  Returns (status, seg_state, seg_gate_prod).
std::tuple<int64_t, at::Tensor, at::Tensor> segment_fwd(const at::Tensor& a_, const at::Tensor& v_,
                                                        int64_t mode, at::Tensor workspace) {
    const at::Tensor a = seq("gate_logit", a_, nullptr);
    const at::Tensor v = seq("value", v_, &a);
    const int64_t B = a.size(0), T = a.size(1), H = a.size(2), Dh = a.size(3);
    const c10::Device dev = a.device();
    check_workspace(workspace, dev);
    const auto opts = a.options().dtype(at::kFloat);
    at::Tensor seg_state = at::empty({B, H, Dh}, opts), seg_prod = at::empty({B, H, Dh}, opts);
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t s = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int st = esa_scan_segment_fwd(B, T, H, Dh, dtype_code(a.scalar_type()), (int)mode,
                                        a.data_ptr(), v.data_ptr(), seg_state.data_ptr<float>(),
                                        seg_prod.data_ptr<float>(), workspace.data_ptr(),
                                        workspace.nbytes(), s);
    return {st, seg_state, seg_prod};
}

// esa_scan_segment_bwd.  Returns (status, seg_d_init).
std::tuple<int64_t, at::Tensor> segment_bwd(const at::Tensor& a_, const at::Tensor& v_,
                                            const at::Tensor& q_, const at::Tensor& dy_,
                                            const c10::optional<at::Tensor>& init_state_,
                                            const c10::optional<at::Tensor>& ckpt_, int64_t mode,
                                            at::Tensor workspace) {
    const at::Tensor a = seq("gate_logit", a_, nullptr);
    const at::Tensor v = seq("value", v_, &a);
    const at::Tensor q = seq("query", q_, &a);
    const at::Tensor dy = seq("dy", dy_, &a);
    const int64_t B = a.size(0), T = a.size(1), H = a.size(2), Dh = a.size(3);
    const c10::Device dev = a.device();
    const std::vector<int64_t> sshape{B, H, Dh};
    const auto init_state = state("init_state", init_state_, sshape, dev);
    check_workspace(workspace, dev);
    c10::optional<at::Tensor> ckpt;
    if (ckpt_.has_value()) {
        TORCH_CHECK_VALUE(ckpt_->scalar_type() == at::kFloat && ckpt_->device() == dev &&
                              (size_t)ckpt_->numel() * 4 >= esa_scan_ckpt_bytes(B, T, H, Dh),
                          "ckpt must be the fp32 checkpoint of scan_fwd(return_ckpt=True)");
        ckpt = ckpt_->contiguous();
    }
    at::Tensor seg_d_init = at::empty(sshape, a.options().dtype(at::kFloat));
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t s = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int st = esa_scan_segment_bwd(
        B, T, H, Dh, dtype_code(a.scalar_type()), (int)mode, a.data_ptr(), v.data_ptr(),
        q.data_ptr(), static_cast<const float*>(ptr(init_state)), dy.data_ptr(),
        static_cast<const float*>(ptr(ckpt)), seg_d_init.data_ptr<float>(), workspace.data_ptr(),
        workspace.nbytes(), s);
    return {st, seg_d_init};
}

// esa_segment_compose over fp32 [nseg, B, H, Dh] stacks.  Returns (status, carry, total).
std::tuple<int64_t, at::Tensor, at::Tensor> segment_compose(const at::Tensor& prod_,
                                                            const at::Tensor& agg_,
                                                            const c10::optional<at::Tensor>& boundary,
                                                            bool reverse) {
    for (const at::Tensor* t : {&prod_, &agg_})
        TORCH_CHECK_VALUE(t->is_cuda() && t->scalar_type() == at::kFloat && t->dim() >= 1,
                          "seg_gate_prod and seg_agg must be fp32 CUDA (HIP) tensors");
    TORCH_CHECK_VALUE(agg_.sizes() == prod_.sizes() && agg_.device() == prod_.device(),
                      "seg_gate_prod and seg_agg must share shape and device");
    const at::Tensor p = prod_.contiguous(), x = agg_.contiguous();
    const c10::Device dev = p.device();
    const at::IntArrayRef lane_shape = p.sizes().slice(1);
    if (boundary.has_value()) out("boundary", *boundary, lane_shape, at::kFloat, dev);
    at::Tensor carry = at::empty_like(p);
    at::Tensor total = at::empty(lane_shape, p.options());
    const int64_t nseg = p.size(0), lanes = nseg ? p.numel() / nseg : 0;
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t s = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int st = esa_segment_compose(nseg, lanes, reverse ? 1 : 0, p.data_ptr<float>(),
                                       x.data_ptr<float>(),
                                       static_cast<const float*>(ptr(boundary)),
                                       carry.data_ptr<float>(), total.data_ptr<float>(), s);
    return {st, carry, total};
}

// esa_state_step: state (fp32 [B, H, Dh], in place) and y ([B, H, Dh], written) from this
// token's gate logits a, values v and queries q ([B, H, Dh], one storage dtype).  Mismatched
// arguments raise ValueError.  Returns the library's status.
int64_t state_step(at::Tensor state_, const at::Tensor& a, const at::Tensor& v,
                   const at::Tensor& q, at::Tensor y, int64_t mode) {
    TORCH_CHECK_VALUE(state_.is_cuda() && state_.scalar_type() == at::kFloat &&
                          state_.dim() == 3 && state_.is_contiguous(),
                      "state must be a contiguous fp32 [B, H, Dh] CUDA (HIP) tensor");
    const at::ScalarType st = a.scalar_type();
    const int code = dtype_code(st);
    TORCH_CHECK_VALUE(code >= 0, "dtype ", st, " not supported");
    const c10::Device dev = state_.device();
    for (const at::Tensor* t : {&a, &v, &q, static_cast<const at::Tensor*>(&y)})
        TORCH_CHECK_VALUE(t->sizes() == state_.sizes() && t->scalar_type() == st &&
                              t->device() == dev && t->is_contiguous(),
                          "step tensors must be contiguous ", st, " ", state_.sizes(), " on ",
                          dev, " like the state");
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t stream = c10::hip::getCurrentHIPStream(dev.index()).stream();
    return esa_state_step(state_.size(0), state_.size(1), state_.size(2), code,
                          static_cast<int>(mode), a.data_ptr(), v.data_ptr(), q.data_ptr(),
                          state_.data_ptr<float>(), y.data_ptr(), stream);
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m) {
    m.def("scan_fwd", &scan_fwd, "esa_scan_fwd on torch tensors (see include/esa.h)");
    m.def("scan_bwd", &scan_bwd, "esa_scan_bwd on torch tensors (see include/esa.h)");
    m.def("state_step", &state_step, "esa_state_step on torch tensors (see include/esa.h)");
    m.def("segment_fwd", &segment_fwd, "esa_scan_segment_fwd on torch tensors");
    m.def("segment_bwd", &segment_bwd, "esa_scan_segment_bwd on torch tensors");
    m.def("segment_compose", &segment_compose, "esa_segment_compose on torch tensors");
}
