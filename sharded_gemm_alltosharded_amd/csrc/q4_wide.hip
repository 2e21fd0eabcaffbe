// The 4-bit streaming kernel (q4_stream.h) for 17 to 32 tokens: three or four
// 8-token blocks.  These instantiations live in a source of their own because
// they are built with the VGPR form of the MFMA (-mllvm
// -amdgpu-mfma-vgpr-form).  With the default register choice the MFMAs write
// the accumulation registers and every 64-input group copies the 16 results to
// ordinary registers for its scale FMAs, about half of the loop's vector
// instructions; the VGPR form removes the copies (decode-MLP gate|up at 24
// tokens 25.4 -> 23.1 us, at 32 tokens 27.1 -> 25.7 us).  With one or two
// 8-token blocks (q4.hip) the same form measured slower (16 tokens: 20.7 ->
// 28.3 us) or no faster, so those keep the default.
#include "q4_stream.h"

namespace sg {

template <bool F16>
hipError_t launch_q4_wide(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    return sh.TB == 3 ? launch_tb<3, F16>(p, s, sh) : launch_tb<4, F16>(p, s, sh);
}

template hipError_t launch_q4_wide<true>(const Problem&, hipStream_t, const Q4Shape&);
template hipError_t launch_q4_wide<false>(const Problem&, hipStream_t, const Q4Shape&);

}  // namespace sg
