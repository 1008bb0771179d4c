// Real spherical harmonics up to degree 3 in the Gaussian-splatting sign and order
// convention (gsplat's colour model, which the gmesh README's Gaussians use), with
// the constants as closed forms.  Internal to libgm.
#pragma once

namespace gm {

constexpr float SH_C0 = 0.28209479177387814f;   // 1/(2 sqrt(pi))
constexpr float SH_C1 = 0.48860251190291992f;   // sqrt(3/(4 pi))
constexpr float SH_C2A = 1.0925484305920792f;   // (1/2) sqrt(15/pi)
constexpr float SH_C2B = 0.31539156525252005f;  // (1/4) sqrt(5/pi)
constexpr float SH_C2C = 0.54627421529603959f;  // (1/4) sqrt(15/pi)
constexpr float SH_C3A = 0.59004358992664352f;  // (1/4) sqrt(35/(2 pi))
constexpr float SH_C3B = 2.8906114426405538f;   // (1/2) sqrt(105/pi)
constexpr float SH_C3C = 0.45704579946446572f;  // (1/4) sqrt(21/(2 pi))
constexpr float SH_C3D = 0.37317633259011546f;  // (1/4) sqrt(7/pi)
constexpr float SH_C3E = 1.4453057213202769f;   // (1/4) sqrt(105/pi)

// Y[0..15] at the unit direction (x, y, z).
__device__ inline void sh_basis_f(float x, float y, float z, float* Y)
{
    const float xx = x * x, yy = y * y, zz = z * z;
    Y[0] = SH_C0;
    Y[1] = -SH_C1 * y;
    Y[2] = SH_C1 * z;
    Y[3] = -SH_C1 * x;
    Y[4] = SH_C2A * x * y;
    Y[5] = -SH_C2A * y * z;
    Y[6] = SH_C2B * (2.0f * zz - xx - yy);
    Y[7] = -SH_C2A * x * z;
    Y[8] = SH_C2C * (xx - yy);
    Y[9] = -SH_C3A * y * (3.0f * xx - yy);
    Y[10] = SH_C3B * x * y * z;
    Y[11] = -SH_C3C * y * (4.0f * zz - xx - yy);
    Y[12] = SH_C3D * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
    Y[13] = -SH_C3C * x * (4.0f * zz - xx - yy);
    Y[14] = SH_C3E * z * (xx - yy);
    Y[15] = -SH_C3A * x * (xx - 3.0f * yy);
}

// Gradient of basis function k with respect to (x, y, z), the polynomial above
// differentiated with the direction components taken as independent.
__device__ inline void sh_basis_grad_f(int k, float x, float y, float z, float& gx, float& gy, float& gz)
{
    const float xx = x * x, yy = y * y, zz = z * z;
    switch (k) {
    case 1: gx = 0.0f; gy = -SH_C1; gz = 0.0f; break;
    case 2: gx = 0.0f; gy = 0.0f; gz = SH_C1; break;
    case 3: gx = -SH_C1; gy = 0.0f; gz = 0.0f; break;
    case 4: gx = SH_C2A * y; gy = SH_C2A * x; gz = 0.0f; break;
    case 5: gx = 0.0f; gy = -SH_C2A * z; gz = -SH_C2A * y; break;
    case 6: gx = -2.0f * SH_C2B * x; gy = -2.0f * SH_C2B * y; gz = 4.0f * SH_C2B * z; break;
    case 7: gx = -SH_C2A * z; gy = 0.0f; gz = -SH_C2A * x; break;
    case 8: gx = 2.0f * SH_C2C * x; gy = -2.0f * SH_C2C * y; gz = 0.0f; break;
    case 9: gx = -6.0f * SH_C3A * x * y; gy = -3.0f * SH_C3A * (xx - yy); gz = 0.0f; break;
    case 10: gx = SH_C3B * y * z; gy = SH_C3B * x * z; gz = SH_C3B * x * y; break;
    case 11: gx = 2.0f * SH_C3C * x * y; gy = -SH_C3C * (4.0f * zz - xx - 3.0f * yy); gz = -8.0f * SH_C3C * y * z; break;
    case 12: gx = -6.0f * SH_C3D * x * z; gy = -6.0f * SH_C3D * y * z; gz = SH_C3D * (6.0f * zz - 3.0f * xx - 3.0f * yy); break;
    case 13: gx = -SH_C3C * (4.0f * zz - 3.0f * xx - yy); gy = 2.0f * SH_C3C * x * y; gz = -8.0f * SH_C3C * x * z; break;
    case 14: gx = 2.0f * SH_C3E * x * z; gy = -2.0f * SH_C3E * y * z; gz = SH_C3E * (xx - yy); break;
    case 15: gx = -3.0f * SH_C3A * (xx - yy); gy = 6.0f * SH_C3A * x * y; gz = 0.0f; break;
    default: gx = 0.0f; gy = 0.0f; gz = 0.0f; break;
    }
}

}  // namespace gm
