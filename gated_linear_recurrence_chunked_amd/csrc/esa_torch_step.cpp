// The decode step's call path from Python without ctypes: torch tensors in, esa_state_step
// out.  Argument marshalling only (shape, dtype, device and layout checks, the current HIP
// stream of the tensors' device); the step itself is the library's kernel behind the C ABI.
// A Python-side loop of one-token steps is host-bound, and this path takes about 2 us of
// host time off every step against the ctypes call and its Python checks.
#include <torch/extension.h>

#include <c10/hip/HIPGuard.h>
#include <c10/hip/HIPStream.h>

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

// One-token update: state (fp32 [B, H, Dh], in place) and y ([B, H, Dh], written) from this
// token's gate logits a, values v and queries q ([B, H, Dh], one storage dtype).  mode is the
// recurrence form (ESA_DIRECT or ESA_CONTROLLED).  Mismatched arguments raise ValueError.
at::Tensor state_step(at::Tensor state, const at::Tensor& a, const at::Tensor& v,
                      const at::Tensor& q, at::Tensor y, int64_t mode) {
    TORCH_CHECK_VALUE(state.is_cuda() && state.scalar_type() == at::kFloat && state.dim() == 3 &&
                          state.is_contiguous(),
                      "state must be a contiguous fp32 [B, H, Dh] CUDA (HIP) tensor");
    const at::ScalarType st = a.scalar_type();
    const int code = dtype_code(st);
    TORCH_CHECK_VALUE(code >= 0, "dtype ", st, " not supported");
    const c10::Device dev = state.device();
    for (const at::Tensor* t : {&a, &v, &q, static_cast<const at::Tensor*>(&y)})
        TORCH_CHECK_VALUE(t->sizes() == state.sizes() && t->scalar_type() == st &&
                              t->device() == dev && t->is_contiguous(),
                          "step tensors must be contiguous ", st, " ", state.sizes(), " on ",
                          dev, " like the state");
    const c10::hip::HIPGuard guard(dev.index());
    const hipStream_t stream = c10::hip::getCurrentHIPStream(dev.index()).stream();
    const int rc = esa_state_step(state.size(0), state.size(1), state.size(2), code,
                                  static_cast<int>(mode), a.data_ptr(), v.data_ptr(),
                                  q.data_ptr(), state.data_ptr<float>(), y.data_ptr(), stream);
    TORCH_CHECK(rc == ESA_OK, "esa_state_step: ", esa_status_string(rc));
    return y;
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m) {
    m.def("state_step", &state_step, "esa_state_step on torch tensors (see include/esa.h)");
}
