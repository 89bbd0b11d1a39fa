// Fast path of the Python binding's gemm_tn(): reads the tensors' dtype,
// device, shape and strides in C++ and calls gemm_tn_ex of the C ABI
// (include/gemm_tn.h) through a pointer the package hands over at import,
// so both paths call the one loaded library.  Argument marshalling only.
// Anything outside the plain cases (wrong dtypes, host tensors, shapes that
// do not match, operands with no unit stride) returns -1 and the Python
// path checks the call and raises; otherwise the library's status is
// returned.
#include <torch/extension.h>

#include <cstdint>

#include "gemm_tn.h"

namespace {

using GemmTnEx = int (*)(int64_t, int64_t, int64_t, int64_t, float,
                         const void *, int, int64_t, int64_t, const void *,
                         int, int64_t, int64_t, float, const void *, int64_t,
                         int64_t, void *, int64_t, int64_t, int, void *);
GemmTnEx g_gemm_tn_ex = nullptr;

void set_entry(int64_t fn)
{
    g_gemm_tn_ex = reinterpret_cast<GemmTnEx>(static_cast<intptr_t>(fn));
}

// (layout, row stride, batch stride) of an fp16 operand with unit stride
// along K (GEMM_TN_ROW_K) or along M / N (GEMM_TN_ROW_MN); false if neither.
bool operand(const at::Tensor &t, int &layout, int64_t &ld, int64_t &bs)
{
    const int64_t nd = t.dim();
    const int64_t rows = t.size(nd - 2), k = t.size(nd - 1);
    const int64_t s_row = t.stride(nd - 2), s_k = t.stride(nd - 1);
    bs = nd == 3 ? t.stride(0) : 0;
    if (k <= 1 || s_k == 1) {
        layout = GEMM_TN_ROW_K;
        ld = rows > 1 ? s_row : (k > 1 ? k : 1);
        return true;
    }
    if (rows <= 1 || s_row == 1) {
        layout = GEMM_TN_ROW_MN;
        ld = s_k;
        return true;
    }
    return false;
}

// Row and batch stride of a row-major C / D; false without unit element
// stride along N.
bool matrix(const at::Tensor &t, int64_t &ld, int64_t &bs)
{
    const int64_t nd = t.dim();
    const int64_t rows = t.size(nd - 2), n = t.size(nd - 1);
    if (n > 1 && t.stride(nd - 1) != 1)
        return false;
    ld = rows > 1 ? t.stride(nd - 2) : (n > 1 ? n : 1);
    bs = nd == 3 ? t.stride(0) : 0;
    return true;
}

int64_t gemm_tn_fast(const at::Tensor &A, const at::Tensor &B,
                     const at::Tensor &D, double alpha, double beta,
                     const c10::optional<at::Tensor> &C, int64_t stream)
{
    if (g_gemm_tn_ex == nullptr)
        return -1;
    const int64_t nd = A.dim();
    if ((nd != 2 && nd != 3) || B.dim() != nd || D.dim() != nd)
        return -1;
    if (A.scalar_type() != at::kHalf || B.scalar_type() != at::kHalf ||
        !A.is_cuda() || !B.is_cuda() || !D.is_cuda())
        return -1;
    const bool d_f32 = D.scalar_type() == at::kFloat;
    if (!d_f32 && D.scalar_type() != at::kHalf)
        return -1;
    const int64_t batch = nd == 3 ? A.size(0) : 1;
    const int64_t M = A.size(nd - 2), K = A.size(nd - 1);
    const int64_t N = B.size(nd - 2);
    if (B.size(nd - 1) != K || (nd == 3 && B.size(0) != batch))
        return -1;
    if (D.size(nd - 2) != M || D.size(nd - 1) != N ||
        (nd == 3 && D.size(0) != batch))
        return -1;
    int la, lb;
    int64_t lda, ldb, sa, sb, ldd, sd;
    if (!operand(A, la, lda, sa) || !operand(B, lb, ldb, sb) ||
        !matrix(D, ldd, sd))
        return -1;
    const void *c_ptr = nullptr;
    int64_t ldc = N, sc = 0;
    if (beta != 0.0) {
        if (!C.has_value())
            return -1;
        const at::Tensor &Ct = *C;
        if (Ct.dim() != nd || Ct.scalar_type() != D.scalar_type() ||
            !Ct.is_cuda() || Ct.sizes() != D.sizes() || !matrix(Ct, ldc, sc))
            return -1;
        c_ptr = Ct.data_ptr();
    }
    return g_gemm_tn_ex(batch, M, N, K, (float)alpha, A.data_ptr(), la, lda,
                        sa, B.data_ptr(), lb, ldb, sb, (float)beta, c_ptr, ldc,
                        sc, D.data_ptr(), ldd, sd,
                        d_f32 ? GEMM_TN_F32 : GEMM_TN_F16,
                        reinterpret_cast<void *>(
                            static_cast<intptr_t>(stream)));
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m)
{
    m.def("set_entry", &set_entry);
    m.def("gemm_tn_fast", &gemm_tn_fast);
}
