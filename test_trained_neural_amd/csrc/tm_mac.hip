// Memory-side wiring of memory-as-context (MAC) on CDNA4 (gfx950): the
// attention window of a segment and the gate of its output ("Titans,
// explained", step 8; "Attack of the Titans", Technical Details, memory as a
// context).  Each segment's tokens query the memory; the recalled vectors go
// between the persistent tokens and the segment itself to form the window
// that attention runs over; the attention output is written into the memory
// and gates the final output through the memory's read of it.  Attention and
// every trained weight stay with the caller; the reads and the write are the
// memory's own calls.  Both kernels move bytes only (HBM-bound): 16-byte
// pieces per thread, grid-strided.
#include "tm_device.h"

namespace tmk {

// window[b] = [persistent (shared over the batch); recalled[b] rounded to the
// operand type; segment[b]], rows of D.
template <class T>
__global__ __launch_bounds__(256) void mac_window_kernel(MacArgs a) {
    constexpr int V = 16 / sizeof(T);            // elements per 16-byte piece
    const int pr = a.D / V;                       // pieces per row
    const int rows = a.P + 2 * a.S;
    const long total = (long)a.B * rows * pr;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int c = (int)(i % pr) * V;
        const long br = i / pr;
        const int r = (int)(br % rows);
        const int b = (int)(br / rows);
        T* dst = reinterpret_cast<T*>(a.out) + br * a.D + c;
        if (r < a.P) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const T*>(a.persistent) + (long)r * a.D + c);
        } else if (r < a.P + a.S) {
            const float* src = a.recalled + ((long)b * a.S + (r - a.P)) * a.D + c;
            if constexpr (sizeof(T) == 2) {
                const f32x8 x = ld8(src);
                *reinterpret_cast<bf16x8*>(dst) = to_bf16(x);
            } else {
                *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
            }
        } else {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const T*>(a.segment) + ((long)b * a.S + (r - a.P - a.S)) * a.D + c);
        }
    }
}

// out = y * mem element-wise, fp32 (y in the operand type, mem the memory's
// fp32 read of y), 4 elements per thread and step.
template <class T>
__global__ __launch_bounds__(256) void mac_gate_kernel(MacArgs a) {
    const long total4 = (long)a.B * a.S * a.D / 4;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total4; i += (long)gridDim.x * 256) {
        const T* y = reinterpret_cast<const T*>(a.segment) + 4 * i;
        const f32x4 m = *reinterpret_cast<const f32x4*>(a.recalled + 4 * i);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)y[e] * m[e];
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + 4 * i) = o;
    }
}

static unsigned mac_blocks(long work) {
    const long b = (work + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

hipError_t launch_mac_window(const MacArgs& a, int f32, hipStream_t st) {
    const long pieces = (long)a.B * (a.P + 2 * a.S) * a.D / (f32 ? 4 : 8);
    if (f32) launch_k(mac_window_kernel<float>, dim3(mac_blocks(pieces)), dim3(256), 0, st, a);
    else launch_k(mac_window_kernel<bf16>, dim3(mac_blocks(pieces)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_mac_gate(const MacArgs& a, int f32, hipStream_t st) {
    const long work = (long)a.B * a.S * a.D / 4;
    if (f32) launch_k(mac_gate_kernel<float>, dim3(mac_blocks(work)), dim3(256), 0, st, a);
    else launch_k(mac_gate_kernel<bf16>, dim3(mac_blocks(work)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace tmk
